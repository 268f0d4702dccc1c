"""bench.py's command line on the CPU: it measures one GPU only, and says so
when asked for more (exit status 2, before touching a device)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="4", RANK="0", LOCAL_RANK="0")
    r = _bench("--gpus", "1", env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_slices_reassemble_the_whole_oracle_call():
    """The CPU baseline times the oracle on independent (sequence, kv-head)
    slices; put back together they must be exactly the whole call's output."""
    import numpy as np

    import bench
    import oracle
    import workloads
    dec = workloads.make_case(3, 12, 4, 64, 200, [200, 17, 0], seed=31)
    chk = workloads.make_case(2, 6, 2, 128, 300, [250, 3], T=5, seed=32)
    bench._ORACLE_INPUTS.update({"dec": [dec], "chk": [chk]})
    try:
        whole = oracle.decode_attention(dec["q"], dec["k"], dec["v"], dec["lens"], dec["scale"])
        parts = np.zeros_like(whole)
        for b in range(3):
            for h in range(4):
                parts[b:b + 1, 3 * h:3 * h + 3] = bench._oracle_slice(("dec", 0, b, h, h + 1, None))
        assert np.array_equal(parts, whole)
        # a length override replays the same cache at another length
        short = oracle.decode_attention(dec["q"][:1], dec["k"][:1], dec["v"][:1], [50], dec["scale"])
        assert np.array_equal(bench._oracle_slice(("dec", 0, 0, 0, 4, 50)), short)
        whole = oracle.chunk_attention(chk["q"], chk["k"], chk["v"], chk["lens"], chk["scale"])
        parts = np.zeros_like(whole)
        for b in range(2):
            for h in range(2):
                parts[b:b + 1, :, 3 * h:3 * h + 3] = bench._oracle_slice(("chk", 0, b, h, h + 1, None))
        assert np.array_equal(parts, whole)
    finally:
        bench._ORACLE_INPUTS.clear()
