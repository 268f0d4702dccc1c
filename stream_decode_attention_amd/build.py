"""Builds libdecattn.so in-tree with hipcc for gfx950.

    python -m stream_decode_attention_amd.build [--verbose]

``--verbose`` adds the compiler's per-kernel resource report (VGPRs, spills,
LDS, occupancy).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "decattn.hip")
LIB = os.path.join(PKG_DIR, "libdecattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fused multiply-add in the kernels is written out; no other contraction
    "-ffp-contract=off",
    # no packed fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the leading scalar kernel arguments (up to 11, within the 16 SGPRs the
    # hardware preloads) are preloaded into SGPRs at wave launch instead of
    # being read from the kernel-argument segment first: about 0.2 us less per
    # launch of the merge kernel on MI355X
    "-mllvm", "-amdgpu-kernarg-preload-count=11",
    "-I", os.path.join(ROOT, "include"),
]


def build_library(verbose: bool = False) -> str:
    """Compile the HIP sources into libdecattn.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, SRC]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="--verbose" in sys.argv))
