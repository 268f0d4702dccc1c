"""HIP prefill_attn (causal attention of many query tokens on the matrix cores)
vs the fp64 oracle on the same seeded bytes, through the C ABI.

prefill_attn computes the chunk operation (token i attends keys
j < ctx + i + 1) for any T, so the reference is oracle.chunk_attention, or,
for sampled rows of full-size calls, oracle.decode_attention at length
ctx + i + 1 (the oracle's pinned chunk == sequential-decodes identity).
Tolerances as everywhere: fp32 output max-abs 1e-4, bf16 output 1e-2 (beyond
that, adjacent to the exact value); rows with no key output exact zeros, and
NaN-poisoned cache slots past ctx + T never reach an output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads
from workloads import BF16_NAN
from tests.gpu_util import assert_bf16_close, assert_f32_close, bits_of, dev_bits, dev_lens, workspace

pytestmark = pytest.mark.gpu


def _run(c, out_dtype=torch.float32, tensors=None):
    q, k, v = tensors if tensors is not None else (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    B, T, Hq, D = q.shape
    out = torch.empty((B, T, Hq, D), dtype=out_dtype, device="cuda")
    sda.prefill_attn(q, k, v, dev_lens(c["lens"]), c["scale"], out)
    torch.cuda.synchronize()
    return out


def _poison_past(c, T):
    """NaN in every cache slot at or past ctx + T (never attended)."""
    k, v = c["k"].copy(), c["v"].copy()
    S = k.shape[2]
    for b, ctx in enumerate(c["lens"]):
        lo = max(0, min(int(ctx) + T, S))
        k[b, :, lo:] = BF16_NAN
        v[b, :, lo:] = BF16_NAN
    return dict(c, k=k, v=v)


CASES = {
    # name: B, T, Hq, Hkv, D, S_max, ctx
    "smollm2-g3-prompt": (1, 300, 15, 5, 64, 512, [0]),
    "tinyllama-g8-chunked": (1, 257, 32, 4, 64, 1024, [100]),
    "llama3-8b-g4-ragged-ctx": (2, 200, 32, 8, 128, 600, [0, 333]),
    "llama3.2-3b-g3-long-ctx": (1, 130, 24, 8, 128, 4096, [3000]),
    "mha-g1": (2, 70, 4, 4, 128, 200, [5, 0]),
    "g2-d64": (3, 97, 8, 4, 64, 256, [0, 64, 159]),
    "one-token": (2, 1, 32, 8, 128, 300, [0, 299]),
    "t-equals-s-max": (1, 256, 8, 2, 128, 256, [0]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_matches_oracle(name):
    B, T, Hq, Hkv, D, S, ctx = CASES[name]
    print(f"prefill case {name}", flush=True)
    c = _poison_past(workloads.make_case(B, Hq, Hkv, D, S, ctx, T=T, seed=200 + sorted(CASES).index(name)), T)
    if T == 1:
        c["q"] = c["q"].reshape(B, 1, Hq, D)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(_run(c, torch.float32), ref)
    assert_bf16_close(_run(c, torch.bfloat16), ref)


def test_prefill_rows_without_keys_and_clamped_limits():
    """ctx < 0 leaves the first rows with no key (zeros); ctx + T > S_max
    clamps the last rows' limits to S_max."""
    B, T, Hq, Hkv, D, S = 2, 120, 8, 2, 128, 160
    c = workloads.make_case(B, Hq, Hkv, D, S, [-40, 100], T=T, seed=230)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    out = _run(c, torch.float32)
    assert_f32_close(out, ref)
    got = out.cpu().numpy()
    assert np.all(got[0, :40] == 0.0)


def test_prefill_equals_chunk_attn_at_small_t():
    """At T <= 16 both entry points serve the same operation."""
    c = workloads.make_case(1, 24, 8, 128, 9000, [8192], T=6, seed=231)
    pre = _run(c, torch.float32)
    ws = workspace(1, 6, 24, 8, 128, 9000)
    ch = torch.empty_like(pre)
    sda.chunk_attn(dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]), dev_lens(c["lens"]), c["scale"], ch, ws)
    torch.cuda.synchronize()
    assert float((pre - ch).abs().max()) <= 2e-4


def _sampled_rows(T, n):
    rows = set([0, 1, 31, 32, 63, 64, T - 1, T - 2, T // 2])
    rng = np.random.default_rng(T)
    rows.update(rng.integers(0, T, size=n).tolist())
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("ctx", [0, 8192])
def test_prefill_full_size_sampled_rows(ctx):
    """Llama-3-8B-shaped prefill of T = 4096 tokens (on an empty cache, and as
    a chunk after 8192 tokens of context): sampled rows against the oracle's
    decode at length ctx + i + 1, every output finite."""
    B, T, Hq, Hkv, D, S = 1, 4096, 32, 8, 128, 16384
    q = workloads.bf16_randn((B, T, Hq, D), 241)
    k = workloads.bf16_randn((B, Hkv, S, D), 242)
    v = workloads.bf16_randn((B, Hkv, S, D), 243)
    scale = float(np.float32(1 / np.sqrt(D)))
    c = {"q": q, "k": k, "v": v, "lens": np.array([ctx], dtype=np.int32), "scale": scale}
    out32, out16 = _run(c, torch.float32), _run(c, torch.bfloat16)
    assert bool(torch.isfinite(out32).all()) and bool(torch.isfinite(out16.float()).all())
    for i in _sampled_rows(T, 24):
        ref = oracle.decode_attention(q[:, i], k, v, np.array([ctx + i + 1], dtype=np.int32), scale)
        assert_f32_close(out32[:, i], ref)
        assert_bf16_close(out16[:, i], ref)


def test_prefill_graph_replay_after_ctx_change():
    B, T, Hq, Hkv, D, S = 2, 100, 16, 4, 64, 400
    c = workloads.make_case(B, Hq, Hkv, D, S, [0, 50], T=T, seed=244)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens(c["lens"])
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sda.prefill_attn(q, k, v, lens, c["scale"], out, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            sda.prefill_attn(q, k, v, lens, c["scale"], out, stream=s)
    for ctx in ([0, 50], [200, 7], [300, 299]):
        with torch.cuda.stream(s):
            lens.copy_(dev_lens(ctx))
            g.replay()
        s.synchronize()
        ref = oracle.chunk_attention(c["q"], c["k"], c["v"], np.array(ctx, dtype=np.int32), c["scale"])
        assert_f32_close(out, ref)
