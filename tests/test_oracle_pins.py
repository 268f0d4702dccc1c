"""Pins for the fp64 oracle: what the pages and the mathematics fix (CPU only).

The pages print no numeric attention example, so the oracle is pinned by
(i) brute force on tiny inputs, (ii) a library routine (PyTorch's fp64
scaled_dot_product_attention, the routine tinydecode's chunk path calls),
(iii) closed forms and invariants the pages state or imply, and (iv) mutation
tests: plausible mistakes planted in a copy of the oracle must each fail one of
these pins.
"""
from __future__ import annotations

import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle.bf16 import bf16_bracket, f64_to_bf16_bits_rne
from tests.oracle_checks import brute_decode, sdpa_chunk, sdpa_decode
import workloads

RNG = np.random.default_rng(20261202)


def _case(B, Hq, Hkv, D, S, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    return q, k, v, np.asarray(lens)


# ---------------------------------------------------------------- bf16 handling

def test_bf16_widening_matches_torch():
    bits = RNG.integers(0, 1 << 16, size=200000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                                  # finite patterns only
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref, equal_nan=False)


def test_bf16_rne_matches_torch_on_fp32_values():
    x = RNG.standard_normal(100000).astype(np.float32) * np.float32(7.0)
    # add exact ties: bf16 value + half a bf16 step, representable in fp32
    base = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -3.0])])
    ours = f64_to_bf16_bits_rne(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_bracket_brackets():
    x = RNG.standard_normal(20000) * 10
    lo, hi = bf16_bracket(x)
    vlo = oracle.bf16_bits_to_f64(lo)
    vhi = oracle.bf16_bits_to_f64(hi)
    assert np.all(vlo <= x) and np.all(x <= vhi)
    # adjacent: no bf16 strictly between them
    gap = vhi - vlo
    step = np.abs(vhi - oracle.bf16_bits_to_f64((hi.astype(np.int32) + np.where(x >= 0, 1, -1)).astype(np.uint16)))
    assert np.all((gap == 0) | (gap <= np.maximum(step, np.abs(vlo) * 2 ** -7 * 1.01)))


# ------------------------------------------------------------- decode: pins

@pytest.mark.parametrize("shape", [
    (1, 1, 1, 4, 5, [3]),
    (2, 4, 2, 8, 9, [9, 1]),
    (2, 3, 1, 5, 7, [0, 6]),
    (1, 4, 4, 6, 8, [8]),
])
def test_decode_matches_brute_force(shape):
    B, Hq, Hkv, D, S, lens = shape
    q, k, v, lens = _case(B, Hq, Hkv, D, S, lens, seed=sum(shape[:5]))
    scale = 1 / math.sqrt(D)
    got = oracle.decode_attention_f64(q, k, v, lens, scale)
    ref = brute_decode(q, k, v, lens, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("B,Hq,Hkv,D,S", [(1, 15, 5, 64, 128), (3, 32, 4, 64, 300), (2, 8, 8, 128, 257)])
def test_decode_matches_torch_sdpa_fp64(B, Hq, Hkv, D, S):
    lens = RNG.integers(0, S + 1, size=B)
    lens[0] = S
    q, k, v, lens = _case(B, Hq, Hkv, D, S, lens, seed=B * 1000 + S)
    scale = float(np.float32(1 / math.sqrt(D)))
    got = oracle.decode_attention_f64(q, k, v, lens, scale)
    ref = sdpa_decode(q, k, v, lens, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_bits_wrapper_equals_f64_path():
    c = workloads.make_case(2, 6, 2, 64, 96, [96, 37], seed=7)
    got = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    ref = oracle.decode_attention_f64(oracle.bf16_bits_to_f64(c["q"]), oracle.bf16_bits_to_f64(c["k"]),
                                      oracle.bf16_bits_to_f64(c["v"]), c["lens"],
                                      float(np.float32(c["scale"])))
    assert np.array_equal(got, ref)


def test_rows_subset_matches_full():
    c = workloads.make_case(2, 8, 2, 64, 64, [64, 20], seed=8)
    full = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    rows = [(0, 3), (1, 7), (1, 0)]
    part = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"], rows=rows)
    for b, h in rows:
        assert np.array_equal(part[b, h], full[b, h])


# --------------------------------------------------------- closed forms

def test_single_key_returns_v0_exactly():
    q, k, v, _ = _case(2, 6, 3, 16, 10, [1, 1], seed=11)
    out = oracle.decode_attention_f64(q, k, v, [1, 1], 0.25)
    for b in range(2):
        for h in range(6):
            assert np.array_equal(out[b, h], v[b, h // 2, 0])


def test_identical_keys_give_mean_of_values():
    q, k, v, _ = _case(1, 4, 2, 16, 12, [9], seed=12)
    k[:, :, :, :] = k[:, :, :1, :]
    out = oracle.decode_attention_f64(q, k, v, [9], 0.3)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[0, h // 2, :9].mean(0))) <= 1e-13


def test_zero_scale_gives_mean_of_values():
    q, k, v, _ = _case(1, 4, 4, 16, 12, [7], seed=13)
    out = oracle.decode_attention_f64(q, k, v, [7], 0.0)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[0, h, :7].mean(0))) <= 1e-13


def test_dominant_key_selects_its_value():
    q, k, v, _ = _case(1, 2, 1, 8, 20, [20], seed=14)
    q[0, :] = 1.0
    k[0, 0] = 0.0
    k[0, 0, 13] = 200.0            # score 1600*scale; others ~N(0, 8)
    out = oracle.decode_attention_f64(q, k, v, [20], 1.0)
    assert np.array_equal(out[0, 0], v[0, 0, 13])
    assert np.array_equal(out[0, 1], v[0, 0, 13])


def test_empty_and_clamped_lengths():
    q, k, v, _ = _case(3, 2, 1, 8, 6, [0, 0, 0], seed=15)
    out = oracle.decode_attention_f64(q, k, v, [0, -5, 99], 0.5)
    assert np.all(out[0] == 0) and np.all(out[1] == 0)
    full = oracle.decode_attention_f64(q, k, v, [0, 0, 6], 0.5)
    assert np.array_equal(out[2], full[2])


def test_two_keys_closed_form():
    # scores a, b -> weights e^a/(e^a+e^b) and e^b/(e^a+e^b)
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[0.5, 9.0], [-1.25, 3.0]]]])
    v = np.array([[[[2.0, -1.0], [4.0, 8.0]]]])
    out = oracle.decode_attention_f64(q, k, v, [2], 2.0)
    a, b = 1.0, -2.5
    wa = 1 / (1 + math.exp(b - a))
    wb = 1 - wa
    assert np.max(np.abs(out[0, 0] - np.array([2 * wa + 4 * wb, -wa + 8 * wb]))) <= 1e-15


# ------------------------------------------------ invariants and split/merge

@pytest.mark.parametrize("chunk", [1, 3, 32, 256, 300])
def test_split_kv_merge_equals_flat(chunk):
    S = 300
    lens = [300, 1, 257, 31]
    q, k, v, lens = _case(4, 6, 2, 16, S, lens, seed=16)
    flat = oracle.decode_attention_f64(q, k, v, lens, 0.2)
    split = oracle.split_kv_attention_f64(q, k, v, lens, 0.2, chunk)
    assert np.max(np.abs(flat - split)) <= 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v, lens = _case(2, 8, 2, 16, 40, [40, 17], seed=17)
    gqa = oracle.decode_attention_f64(q, k, v, lens, 0.25)
    mha = oracle.decode_attention_f64(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), lens, 0.25)
    assert np.array_equal(gqa, mha)
    # and not a strided (h % Hkv) grouping
    strided = oracle.decode_attention_f64(q, np.tile(k, (1, 4, 1, 1)), np.tile(v, (1, 4, 1, 1)), lens, 0.25)
    assert np.max(np.abs(gqa - strided)) > 1e-3


def test_batch_rows_independent():
    q, k, v, lens = _case(3, 4, 2, 16, 30, [30, 5, 18], seed=18)
    full = oracle.decode_attention_f64(q, k, v, lens, 0.25)
    for b in range(3):
        one = oracle.decode_attention_f64(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], 0.25)
        assert np.array_equal(one[0], full[b])


def test_linear_in_values():
    q, k, v1, lens = _case(2, 4, 2, 16, 30, [30, 11], seed=19)
    v2 = np.random.default_rng(20).standard_normal(v1.shape)
    a, b = 0.7, -1.9
    lhs = oracle.decode_attention_f64(q, k, a * v1 + b * v2, lens, 0.25)
    rhs = a * oracle.decode_attention_f64(q, k, v1, lens, 0.25) + b * oracle.decode_attention_f64(q, k, v2, lens, 0.25)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12


def test_key_permutation_invariance():
    q, k, v, lens = _case(1, 4, 2, 16, 30, [25], seed=21)
    perm = np.random.default_rng(22).permutation(25)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :25] = k[:, :, perm]
    v2[:, :, :25] = v[:, :, perm]
    a = oracle.decode_attention_f64(q, k, v, lens, 0.25)
    b = oracle.decode_attention_f64(q, k2, v2, lens, 0.25)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_keys_past_length_are_never_read():
    q, k, v, lens = _case(2, 4, 2, 16, 30, [12, 30], seed=23)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 12:] = np.nan
    v2[0, :, 12:] = np.inf
    a = oracle.decode_attention_f64(q, k, v, lens, 0.25)
    b = oracle.decode_attention_f64(q, k2, v2, lens, 0.25)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- chunk

@pytest.mark.parametrize("B,T,Hq,Hkv,D,S,ctx", [
    (1, 6, 24, 8, 32, 64, [40]),
    (2, 3, 4, 2, 16, 20, [0, 17]),
    (1, 4, 3, 1, 8, 10, [8]),        # ctx + T > S_max: later rows clamp
])
def test_chunk_equals_sequential_decodes(B, T, Hq, Hkv, D, S, ctx):
    rng = np.random.default_rng(B * 100 + T)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    out = oracle.chunk_attention_f64(q, k, v, ctx, 0.3)
    for i in range(T):
        lens = np.asarray(ctx) + i + 1
        dec = oracle.decode_attention_f64(q[:, i], k, v, lens, 0.3)
        assert np.max(np.abs(out[:, i] - dec)) <= 1e-12


def test_chunk_matches_sdpa_causal_mask():
    rng = np.random.default_rng(31)
    B, T, Hq, Hkv, D, S = 2, 6, 24, 8, 32, 80
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    ctx = np.array([70, 3])
    out = oracle.chunk_attention_f64(q, k, v, ctx, 0.125)
    ref = sdpa_chunk(q, k, v, ctx, 0.125)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("ctx", [[0, 0], [0, 37], [-5, 150]])
def test_prefill_length_chunk_matches_sdpa_and_torch_causal(ctx):
    """T in the hundreds (prefill): the explicit-mask SDPA reference, and at
    ctx = 0 torch's own is_causal path, which knows nothing of the offsets."""
    rng = np.random.default_rng(32)
    B, T, Hq, Hkv, D, S = 2, 160, 8, 2, 16, 200
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    ctx = np.array(ctx)
    out = oracle.chunk_attention_f64(q, k, v, ctx, 0.25)
    # rows with no key (ctx + i + 1 <= 0) are zeros; compare the others
    live = (ctx[:, None] + np.arange(T)[None, :] + 1) > 0
    ref = sdpa_chunk(q, k, v, ctx, 0.25)
    assert np.max(np.abs((out - ref)[live])) <= 1e-12
    assert np.all(out[~live] == 0)
    if not ctx.any():
        qt = torch.as_tensor(q).permute(0, 2, 1, 3)
        kt = torch.as_tensor(k[:, :, :T]).repeat_interleave(Hq // Hkv, dim=1)
        vt = torch.as_tensor(v[:, :, :T]).repeat_interleave(Hq // Hkv, dim=1)
        tc = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
        assert np.max(np.abs(out - tc.permute(0, 2, 1, 3).numpy())) <= 1e-12


def test_chunk_row_unchanged_by_later_key():
    rng = np.random.default_rng(32)
    q = rng.standard_normal((1, 5, 4, 16))
    k = rng.standard_normal((1, 2, 40, 16))
    v = rng.standard_normal((1, 2, 40, 16))
    a = oracle.chunk_attention_f64(q, k, v, [30], 0.25)
    k[0, :, 32] += 5.0                        # key ctx+2: seen by rows i >= 2
    b = oracle.chunk_attention_f64(q, k, v, [30], 0.25)
    assert np.array_equal(a[0, :2], b[0, :2])
    assert np.all(np.max(np.abs(a[0, 2:] - b[0, 2:]), axis=-1) > 0)


def test_chunk_bits_wrapper_equals_f64_path():
    c = workloads.make_case(1, 24, 8, 128, 64, [40], T=6, seed=33)
    got = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    ref = oracle.chunk_attention_f64(oracle.bf16_bits_to_f64(c["q"]), oracle.bf16_bits_to_f64(c["k"]),
                                     oracle.bf16_bits_to_f64(c["v"]), c["lens"], c["scale"])
    assert np.array_equal(got, ref)


# ------------------------------------------------------- mutation tests

def _pin_battery(att) -> list[str]:
    """Run a compact set of the pins above against a (possibly mutated) oracle module.

    Returns the names of the pins that fail.
    """
    failed = []
    # brute force
    q, k, v, lens = _case(2, 4, 2, 8, 9, [9, 4], seed=41)
    try:
        if np.max(np.abs(att.decode_attention_f64(q, k, v, lens, 0.35) - brute_decode(q, k, v, lens, 0.35))) > 1e-12:
            failed.append("brute")
    except Exception:
        failed.append("brute-raised")
    # sdpa
    q, k, v, lens = _case(2, 6, 3, 16, 33, [33, 20], seed=42)
    try:
        if np.max(np.abs(att.decode_attention_f64(q, k, v, lens, 0.25) - sdpa_decode(q, k, v, lens, 0.25))) > 1e-12:
            failed.append("sdpa")
    except Exception:
        failed.append("sdpa-raised")
    # dominant key with a large score
    q, k, v, _ = _case(1, 2, 1, 8, 20, [20], seed=14)
    q[0, :] = 1.0
    k[0, 0] = 0.0
    k[0, 0, 13] = 200.0
    with np.errstate(all="ignore"):
        try:
            o = att.decode_attention_f64(q, k, v, [20], 1.0)
            if not np.array_equal(o[0, 0], v[0, 0, 13]):
                failed.append("dominant")
        except Exception:
            failed.append("dominant-raised")
    # split/merge
    q, k, v, lens = _case(2, 4, 2, 8, 50, [50, 17], seed=43)
    try:
        d = np.max(np.abs(att.split_kv_attention_f64(q, k, v, lens, 0.3, 7) - brute_decode(q, k, v, lens, 0.3)))
        if not d <= 1e-12:
            failed.append("split")
    except Exception:
        failed.append("split-raised")
    # chunk vs sdpa with explicit causal mask
    rng = np.random.default_rng(44)
    qc = rng.standard_normal((1, 4, 6, 8))
    kc = rng.standard_normal((1, 2, 30, 8))
    vc = rng.standard_normal((1, 2, 30, 8))
    try:
        if np.max(np.abs(att.chunk_attention_f64(qc, kc, vc, [20], 0.3) - sdpa_chunk(qc, kc, vc, [20], 0.3))) > 1e-12:
            failed.append("chunk")
    except Exception:
        failed.append("chunk-raised")
    # bf16 widening against torch
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    try:
        if not np.array_equal(att.bf16_bits_to_f64(bits), ref):
            failed.append("bf16")
    except Exception:
        failed.append("bf16-raised")
    return failed


MUTANTS = {
    "gqa-strided-mapping": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "dropped-max-subtraction": ("np.exp(scores - scores.max())", "np.exp(scores)"),
    "dropped-normalisation": ("return (w @ V) / w.sum()", "return (w @ V)"),
    "dropped-scale": ("s = float(scale) * (K @ q[b, h])\n            out[b, h] = _softmax_weighted_sum(s, V)\n    return out\n\n\ndef decode_attention(",
                      "s = (K @ q[b, h])\n            out[b, h] = _softmax_weighted_sum(s, V)\n    return out\n\n\ndef decode_attention("),
    "keys-used-as-values": ("return (w @ V) / w.sum()", "return (w @ V[:, ::-1]) / w.sum()"),
    "causal-off-by-one": ("_clamp_len(ctx + i + 1, S_max)", "_clamp_len(ctx + i, S_max)"),
    "merge-weight-sign": ("w = np.exp(np.array(ms) - M)", "w = np.exp(M - np.array(ms))"),
    "merge-dropped-l-weight": ("L = float(np.dot(w, ls))", "L = float(np.sum(ls))"),
    "bf16-shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "length-off-by-one": ("K = np.asarray(k[b, kvh, :n], dtype=np.float64)\n            V = np.asarray(v[b, kvh, :n], dtype=np.float64)\n            s = float(scale)",
                          "K = np.asarray(k[b, kvh, :n - 1], dtype=np.float64)\n            V = np.asarray(v[b, kvh, :n - 1], dtype=np.float64)\n            s = float(scale)"),
    "transposed-chunk-scores": ("S = scale * (q[:, h, :] @ Kh.T)", "S = scale * (q[::-1, h, :] @ Kh.T)"),
}


def _load_mutant(old: str, new: str) -> types.ModuleType:
    src = open(oatt.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_pin_battery_passes_on_oracle():
    assert _pin_battery(oatt) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    mutant = _load_mutant(old, new)
    with np.errstate(all="ignore"):
        failed = _pin_battery(mutant)
    assert failed, f"mutant {name} passed every pin"
