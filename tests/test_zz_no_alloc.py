"""decode_attn_noalloc: the allocation-free variant of decode_attn.

Called through the C ABI (the ctypes binding) and compared with decode_attn on
the same inputs and tile size: the two share their kernels, so the outputs must
be identical bit for bit (and within the oracle's tolerances). Two calls in a
row, the second on a smaller input, check that the static scratch array keeps
no state that matters from one call to the next.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads
from tests.gpu_util import assert_bf16_close, assert_f32_close, dev_bits, dev_lens, run_decode


def _noalloc(c, tensors, out_dtype, chunk=0):
    q, k, v = tensors
    B, Hq, D = q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    sda.decode_attn_noalloc(q, k, v, dev_lens(c["lens"]), c["scale"], out, chunk)
    torch.cuda.synchronize()
    return out


@pytest.mark.gpu
def test_noalloc_equals_decode_attn_on_two_calls_second_smaller():
    # first: the batched ragged Llama-3-8B-shaped decode at a reduced cache
    # (B = 8, Hq 32, Hkv 8, D 128, S_max 8192); second: the SmolLM2-360M head
    # shape on a 4096-slot cache at 1000 keys (a far smaller workspace)
    rng = np.random.default_rng(5)
    big = workloads.make_case(8, 32, 8, 128, 8192, rng.integers(1, 8193, size=8), seed=501)
    small = workloads.make_case(1, 15, 5, 64, 4096, [1000], seed=502)
    for c in (big, small):
        tensors = (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
        ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
        for dt in (torch.float32, torch.bfloat16):
            got = _noalloc(c, tensors, dt)
            want = run_decode(c, tensors=tensors, out_dtype=dt)
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))
            if dt == torch.float32:
                assert_f32_close(got, ref)
            else:
                assert_bf16_close(got, ref)
