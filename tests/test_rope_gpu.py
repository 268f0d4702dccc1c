"""HIP rope_kv_write vs the fp64 oracle on the same seeded bytes, through the C ABI.

Both sides compute every rotated value in fp64 and round it once to the
nearest-even bf16, so the outputs are compared bit for bit. The only allowed
difference is at a near tie: the two fp64 computations (different pow/sincos
implementations) may fall on either side of a bf16 rounding midpoint when the
exact value lies within 1e-9 (relative) of it; such an element must hold one
of the two bf16 neighbours. V is copied and every slot not written keeps its
bytes: both bit-exact, with no exception.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads
from oracle.bf16 import bf16_bracket
from tests.gpu_util import assert_f32_close, bits_of, dev_bits, dev_lens, workspace

pytestmark = pytest.mark.gpu

LLAMA3 = {"factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0, "original_max_position": 8192.0}


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _assert_rounded(got, ref, exact_f64, what):
    """got == ref bit for bit, except near ties of the fp64 value (see module doc)."""
    diff = got != ref
    if not diff.any():
        return 0
    x = exact_f64[diff]
    lo, hi = bf16_bracket(x)
    adjacent = (got[diff] == lo) | (got[diff] == hi)
    mid = (_f64(lo) + _f64(hi)) / 2
    near_tie = np.abs(x - mid) <= 1e-9 * np.abs(x)
    assert adjacent.all() and near_tie.all(), \
        f"{what}: {int(diff.sum())} elements differ, {int((~(adjacent & near_tie)).sum())} not at a near tie"
    return int(diff.sum())


def _inputs(B, T, Hq, Hkv, D, S, seed):
    return (workloads.bf16_randn((B, T, Hq, D), seed * 10 + 1), workloads.bf16_randn((B, T, Hkv, D), seed * 10 + 2),
            workloads.bf16_randn((B, T, Hkv, D), seed * 10 + 3), workloads.bf16_randn((B, Hkv, S, D), seed * 10 + 4),
            workloads.bf16_randn((B, Hkv, S, D), seed * 10 + 5))


def _run_and_check(B, T, Hq, Hkv, D, S, pos0, theta, pairing, llama3, seed, in_place=False):
    q, k, v, kc, vc = _inputs(B, T, Hq, Hkv, D, S, seed)
    dq, dk, dv, dkc, dvc = (dev_bits(x) for x in (q, k, v, kc, vc))
    dq_out = dq if in_place else torch.empty_like(dq)
    sda.rope_kv_write(dq, dk, dv, dev_lens(pos0), dq_out, dkc, dvc, theta, pairing, llama3)
    torch.cuda.synchronize()
    q_ref, kc_ref, vc_ref = oracle.rope_kv_write(q, k, v, pos0, kc, vc, theta=theta, pairing=pairing, llama3=llama3)
    freqs = oracle.model_frequencies(D, theta, llama3)
    pos = oracle.token_positions(pos0, T, S)
    q64, k64 = oracle.rope_kv_write_f64(_f64(q), _f64(k), pos, freqs, pairing)
    ties = _assert_rounded(bits_of(dq_out), q_ref, q64, "q")
    got_kc, got_vc = bits_of(dkc), bits_of(dvc)
    assert np.array_equal(got_vc, vc_ref), "v cache differs"
    # key cache: unwritten slots exact; written slots rounded from the oracle's fp64 keys
    k_exact = _f64(kc_ref).copy()
    for b in range(B):
        for i in range(T):
            p = int(pos[b, i])
            if p < S:
                k_exact[b, :, p] = k64[b, i]
    written = np.zeros((B, 1, S, 1), dtype=bool)
    for b in range(B):
        for p in pos[b]:
            if p < S:
                written[b, 0, p, 0] = True
    assert np.array_equal(np.where(written, 0, got_kc), np.where(written, 0, kc_ref)), "an unwritten key slot changed"
    ties += _assert_rounded(got_kc, kc_ref, k_exact, "k cache")
    return q_ref, kc_ref, vc_ref, dq_out, dkc, dvc, ties


CASES = {
    # name: B, T, Hq, Hkv, D, S_max, pos0, theta, pairing, llama3
    "smollm2-decode-at-last-slot": (1, 1, 15, 5, 64, 4096, [4095], 100000.0, "half", None),
    "tinyllama-decode": (1, 1, 32, 4, 64, 8192, [5000], 10000.0, "half", None),
    "llama3-8b-batch-ragged": (8, 1, 32, 8, 128, 2048, [5, 291, 2047, 0, 1000, 1500, 17, 2046], 500000.0, "half", None),
    "llama3.2-3b-verify-llama3-scaling": (1, 6, 24, 8, 128, 16384, [8192], 500000.0, "half", LLAMA3),
    "adjacent-pairs-d64": (2, 4, 8, 2, 64, 300, [10, 250], 10000.0, "adjacent", None),
    "adjacent-llama3-d128": (3, 3, 12, 4, 128, 100, [0, 50, 97], 500000.0, "adjacent", LLAMA3),
    "past-the-cache-and-clamped": (4, 5, 6, 2, 64, 40, [-7, 37, 40, 1000], 10000.0, "half", None),
    "sixteen-tokens-per-row": (2, 16, 8, 8, 128, 64, [3, 48], 10000.0, "half", LLAMA3),
    "theta-one-all-angles-equal-position": (2, 2, 4, 1, 64, 32, [1, 30], 1.0, "half", None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_rope_kv_write_matches_oracle(name):
    B, T, Hq, Hkv, D, S, pos0, theta, pairing, llama3 = CASES[name]
    print(f"rope case {name}", flush=True)
    _run_and_check(B, T, Hq, Hkv, D, S, pos0, theta, pairing, llama3, seed=100 + sorted(CASES).index(name))


@pytest.mark.parametrize("pairing", ["half", "adjacent"])
def test_rope_in_place(pairing):
    _run_and_check(3, 2, 16, 4, 128, 512, [7, 300, 510], 500000.0, pairing, LLAMA3, seed=31, in_place=True)


def test_rope_position_zero_keeps_bits():
    q, k, v, kc, vc = _inputs(2, 1, 8, 2, 64, 16, seed=32)
    dq, dkc, dvc = dev_bits(q), dev_bits(kc), dev_bits(vc)
    out = torch.empty_like(dq)
    sda.rope_kv_write(dq, dev_bits(k), dev_bits(v), dev_lens([0, 0]), out, dkc, dvc, 10000.0)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), q)
    assert np.array_equal(bits_of(dkc)[:, :, 0], k[:, 0])
    assert np.array_equal(bits_of(dvc)[:, :, 0], v[:, 0])


def test_rope_full_size_batched_decode():
    """Llama-3-8B-shaped batched decode: B=8 rows of a 32768-slot cache at the
    headline's ragged lengths; the whole 1 GB cache pair is compared."""
    c = workloads.make_config(4)
    B, Hq, Hkv, D, S = 8, 32, 8, 128, 32768
    pos0 = np.minimum(c["lens"], S - 1)
    q = workloads.bf16_randn((B, 1, Hq, D), 401)
    k = workloads.bf16_randn((B, 1, Hkv, D), 402)
    v = workloads.bf16_randn((B, 1, Hkv, D), 403)
    dkc, dvc = dev_bits(c["k"]), dev_bits(c["v"])
    dq = dev_bits(q)
    out = torch.empty_like(dq)
    sda.rope_kv_write(dq, dev_bits(k), dev_bits(v), dev_lens(pos0), out, dkc, dvc, 500000.0)
    torch.cuda.synchronize()
    q_ref, kc_ref, vc_ref = oracle.rope_kv_write(q, k, v, pos0, c["k"], c["v"], theta=500000.0)
    freqs = oracle.model_frequencies(D, 500000.0)
    pos = oracle.token_positions(pos0, 1, S)
    q64, k64 = oracle.rope_kv_write_f64(_f64(q), _f64(k), pos, freqs)
    _assert_rounded(bits_of(out), q_ref, q64, "q")
    got_vc = bits_of(dvc)
    assert np.array_equal(got_vc, vc_ref)
    del got_vc, vc_ref
    got_kc = bits_of(dkc)
    diff = np.argwhere(got_kc != kc_ref)
    for b, h, p, d in diff:                     # only written slots may differ, at near ties
        assert p == pos[b, 0], f"slot {(b, h, p)} changed"
        _assert_rounded(got_kc[b, h, p, d:d + 1], kc_ref[b, h, p, d:d + 1], k64[b, 0, h, d:d + 1], "k cache")


def _chunk_out(q_bits, kc, vc, ctx, scale, T):
    B, _, Hq, D = q_bits.shape
    Hkv, S = kc.shape[1], kc.shape[2]
    ws = workspace(B, T, Hq, Hkv, D, S)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    sda.chunk_attn(q_bits, kc, vc, ctx, scale, out, ws)
    torch.cuda.synchronize()
    return out


def test_verify_step_rope_write_then_chunk_attention():
    """Llama-3.2-3B-shaped verify step: rotate and write T = 6 draft tokens at
    ctx 8192, then causal chunk attention over the updated cache."""
    B, T, Hq, Hkv, D, S, ctx = 1, 6, 24, 8, 128, 16384, [8192]
    q, k, v, kc, vc = _inputs(B, T, Hq, Hkv, D, S, seed=33)
    dq, dkc, dvc = dev_bits(q), dev_bits(kc), dev_bits(vc)
    lens = dev_lens(ctx)
    sda.rope_kv_write(dq, dev_bits(k), dev_bits(v), lens, dq, dkc, dvc, 500000.0, "half", LLAMA3)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = _chunk_out(dq, dkc, dvc, lens, scale, T)
    q_ref, kc_ref, vc_ref = oracle.rope_kv_write(q, k, v, ctx, kc, vc, theta=500000.0, llama3=LLAMA3)
    assert np.array_equal(bits_of(dq), q_ref)
    ref = oracle.chunk_attention(q_ref, kc_ref, vc_ref, np.asarray(ctx, dtype=np.int32), scale)
    assert_f32_close(out, ref)


def test_decode_loop_in_a_graph():
    """One captured graph = rope_kv_write then attention over j < pos0 + 1 (a
    T = 1 chunk call); replayed for 5 steps with new q/k/v copied in and the
    device lengths advanced between replays, each step checked."""
    B, Hq, Hkv, D, S = 2, 8, 2, 64, 256
    _, _, _, kc, vc = _inputs(B, 1, Hq, Hkv, D, S, seed=34)
    lens_np = np.array([10, 100], dtype=np.int32)
    dkc, dvc = dev_bits(kc), dev_bits(vc)
    lens = dev_lens(lens_np)
    q_in = torch.empty((B, 1, Hq, D), dtype=torch.int16, device="cuda")
    k_in = torch.empty((B, 1, Hkv, D), dtype=torch.int16, device="cuda")
    v_in = torch.empty_like(k_in)
    q_rot = torch.empty_like(q_in)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    ws = workspace(B, 1, Hq, Hkv, D, S, poison=False)
    scale = 0.125
    s = torch.cuda.Stream()

    def step():
        sda.rope_kv_write(q_in, k_in, v_in, lens, q_rot, dkc, dvc, 10000.0, stream=s)
        sda.chunk_attn(q_rot, dkc, dvc, lens, scale, out, ws, stream=s)

    q0, k0, v0, _, _ = _inputs(B, 1, Hq, Hkv, D, 1, seed=35)
    with torch.cuda.stream(s):
        q_in.copy_(dev_bits(q0)); k_in.copy_(dev_bits(k0)); v_in.copy_(dev_bits(v0))
        step()                                  # warm-up outside the graph (writes slot lens)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
    # the warm-up wrote step 0 already; the reference cache follows the same sequence
    kc_ref, vc_ref = kc, vc
    _, kc_ref, vc_ref = oracle.rope_kv_write(q0, k0, v0, lens_np, kc_ref, vc_ref, theta=10000.0)
    for t in range(5):
        qt, kt, vt, _, _ = _inputs(B, 1, Hq, Hkv, D, 1, seed=40 + t)
        with torch.cuda.stream(s):
            lens.add_(1)
            q_in.copy_(dev_bits(qt)); k_in.copy_(dev_bits(kt)); v_in.copy_(dev_bits(vt))
            g.replay()
        s.synchronize()
        lens_np = lens_np + 1
        q_ref, kc_ref, vc_ref = oracle.rope_kv_write(qt, kt, vt, lens_np, kc_ref, vc_ref, theta=10000.0)
        assert np.array_equal(bits_of(q_rot), q_ref), f"step {t}: rotated q"
        ref = oracle.chunk_attention(q_ref, kc_ref, vc_ref, lens_np, scale)
        assert_f32_close(out, ref)
    assert np.array_equal(bits_of(dkc), kc_ref) and np.array_equal(bits_of(dvc), vc_ref)
