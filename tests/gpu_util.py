"""Helpers for the GPU tests: upload seeded bf16 bytes, call the library, compare."""
from __future__ import annotations

import numpy as np
import torch

import stream_decode_attention_amd as sda
from oracle import bf16_bits_to_f64
from oracle.bf16 import bf16_bracket

F32_TOL = 1e-4     # max-abs error allowed for fp32 output
BF16_TOL = 1e-2    # max-abs error allowed for bf16 output


def dev_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def dev_lens(lens) -> torch.Tensor:
    return torch.as_tensor(np.asarray(lens, dtype=np.int32)).to("cuda")


def workspace(B, T, Hq, Hkv, D, S, chunk=0, poison=True) -> torch.Tensor:
    n = sda.workspace_bytes(B, T, Hq, Hkv, D, S, chunk)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    if poison:
        ws.fill_(0xFF)          # NaN everywhere: a read of an unwritten tile shows up
    return ws


def run_decode(c: dict, *, chunk=0, out_dtype=torch.float32, lens=None, tensors=None):
    q, k, v = tensors if tensors is not None else (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    lens = c["lens"] if lens is None else lens
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    ws = workspace(B, 1, Hq, Hkv, D, S, chunk)
    out = torch.empty((B, Hq, D), dtype=out_dtype, device="cuda")
    sda.decode_attn(q, k, v, dev_lens(lens), c["scale"], out, ws, chunk)
    torch.cuda.synchronize()
    return out


def run_chunk(c: dict, *, chunk=0, out_dtype=torch.float32, tensors=None):
    q, k, v = tensors if tensors is not None else (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    B, T, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    ws = workspace(B, T, Hq, Hkv, D, S, chunk)
    out = torch.empty((B, T, Hq, D), dtype=out_dtype, device="cuda")
    sda.chunk_attn(q, k, v, dev_lens(c["lens"]), c["scale"], out, ws, chunk)
    torch.cuda.synchronize()
    return out


def to_f64(out: torch.Tensor) -> np.ndarray:
    if out.dtype == torch.float32:
        return out.cpu().double().numpy()
    return bf16_bits_to_f64(bits_of(out))


def bits_of(out: torch.Tensor) -> np.ndarray:
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_f32_close(out: torch.Tensor, ref: np.ndarray, tol=F32_TOL, mask=None):
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - ref)
    if mask is not None:
        err = err[mask]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"max abs error {worst:.3e} > {tol}"
    return worst


def assert_bf16_close(out: torch.Tensor, ref: np.ndarray, tol=BF16_TOL, mask=None):
    """bf16 output: max-abs <= tol; an element beyond tol must still be one of
    the two bf16 values adjacent to the fp64 result (the rounding quantum of
    bf16 exceeds tol for |x| >= 4)."""
    bits = bits_of(out)
    got = bf16_bits_to_f64(bits)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - ref)
    sel = np.ones(err.shape, bool) if mask is None else mask
    bad = (err > tol) & sel
    if bad.any():
        lo, hi = bf16_bracket(ref[bad])
        ok = (bits[bad] == lo) | (bits[bad] == hi)
        assert ok.all(), f"{int((~ok).sum())} bf16 outputs off by more than {tol} and not adjacent to the exact value"
    return float(err[sel].max()) if sel.any() else 0.0
