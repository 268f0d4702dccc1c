"""Pins for the rotary-embedding / K/V-write oracle (CPU only).

The pages print no rotary example, so the oracle is pinned by (i) a second
formulation, complex multiplication by e^{i p f}, on NumPy's complex type;
(ii) a brute-force loop over scalars with Python's math module; (iii) closed
forms and invariants of a rotation (identity at position 0, a quarter turn,
pair norms, the relative-position property that defines RoPE); (iv) the llama3
scaling's own region boundaries; and (v) mutation tests: plausible mistakes
planted in a copy of the oracle must each fail one of the pins.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest

import oracle
from oracle import rope as orope
from oracle.bf16 import f64_to_bf16_bits_rne
import workloads

RNG = np.random.default_rng(20261203)
LLAMA3 = {"factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0, "original_max_position": 8192.0}


def _bits(x):
    return f64_to_bf16_bits_rne(np.asarray(x, dtype=np.float64))


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _complex_rotate(x, pos, freqs, pairing):
    """The same rotation as multiplication of complex numbers by e^{i p f}."""
    D = x.shape[-1]
    if pairing == "half":
        z = x[..., : D // 2] + 1j * x[..., D // 2:]
    else:
        z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * (np.asarray(pos, dtype=np.float64)[..., None] * freqs))
    out = np.empty_like(x)
    if pairing == "half":
        out[..., : D // 2], out[..., D // 2:] = z.real, z.imag
    else:
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def _loop_rotate(vec, p, theta, pairing):
    """Brute force for one head vector: scalar loops, Python's math module."""
    D = len(vec)
    out = [0.0] * D
    for j in range(D // 2):
        f = theta ** (-(2.0 * j) / D)
        c, s = math.cos(p * f), math.sin(p * f)
        ia, ib = (j, j + D // 2) if pairing == "half" else (2 * j, 2 * j + 1)
        out[ia] = vec[ia] * c - vec[ib] * s
        out[ib] = vec[ia] * s + vec[ib] * c
    return out


# ------------------------------------------------------------ frequencies

def test_frequencies_closed_form():
    f = oracle.rope_frequencies(128, 10000.0)
    assert f.shape == (64,)
    assert f[0] == 1.0
    assert math.isclose(f[63], 10000.0 ** (-126 / 128), rel_tol=1e-15)
    ratio = f[1:] / f[:-1]
    assert np.allclose(ratio, 10000.0 ** (-2 / 128), rtol=1e-13, atol=0)
    assert np.all(np.diff(f) < 0)


def test_llama3_scaling_regions():
    D, theta = 128, 500000.0
    f = oracle.rope_frequencies(D, theta)
    g = oracle.llama3_scale_frequencies(f, **LLAMA3)
    w = 2 * np.pi / f
    L = LLAMA3["original_max_position"]
    hi_w, lo_w = L / LLAMA3["high_freq_factor"], L / LLAMA3["low_freq_factor"]
    keep, slow = w < hi_w, w > lo_w
    mid = ~keep & ~slow
    assert keep.any() and slow.any() and mid.any()      # the shape exercises all three regions
    assert np.array_equal(g[keep], f[keep])
    assert np.array_equal(g[slow], f[slow] / LLAMA3["factor"])
    assert np.all(g[mid] < f[mid]) and np.all(g[mid] > f[mid] / LLAMA3["factor"])
    # the frequency order is kept (the blend is monotone across the regions)
    assert np.all(np.diff(g) < 0)


def test_llama3_blend_quarter_point_and_boundaries():
    L, lo, hi, fac = 8192.0, 1.0, 4.0, 32.0
    # a frequency with L / wavelength a quarter of the way from lo to hi gets
    # weight 1/4 on the unscaled frequency, 3/4 on the slowed one
    f_q = 2 * np.pi * (lo + 0.25 * (hi - lo)) / L
    g = oracle.llama3_scale_frequencies([f_q], fac, lo, hi, L)[0]
    assert math.isclose(g, 0.75 * f_q / fac + 0.25 * f_q, rel_tol=1e-14)
    # just inside each boundary the blend meets the neighbouring region
    eps = 1e-9
    f_hi = 2 * np.pi * hi / L * (1 - eps)        # wavelength just above L/hi: blend with s ~ 1
    f_lo = 2 * np.pi * lo / L * (1 + eps)        # wavelength just below L/lo: blend with s ~ 0
    g_hi, g_lo = oracle.llama3_scale_frequencies([f_hi, f_lo], fac, lo, hi, L)
    assert math.isclose(g_hi, f_hi, rel_tol=1e-7)
    assert math.isclose(g_lo, f_lo / fac, rel_tol=1e-7)


def test_llama3_factor_one_changes_nothing():
    f = oracle.rope_frequencies(64, 500000.0)
    g = oracle.llama3_scale_frequencies(f, 1.0, 1.0, 4.0, 8192.0)
    assert np.allclose(g, f, rtol=1e-15, atol=0)


# -------------------------------------------------------------- rotation

@pytest.mark.parametrize("pairing", ["half", "adjacent"])
def test_rotation_equals_complex_multiplication(pairing):
    x = RNG.standard_normal((3, 5, 64))
    pos = RNG.integers(0, 40000, size=(3, 5))
    f = oracle.model_frequencies(64, 10000.0)
    got = oracle.rotate_f64(x, pos, f, pairing)
    ref = _complex_rotate(x, pos, f, pairing)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("pairing", ["half", "adjacent"])
def test_rotation_matches_scalar_loops(pairing):
    x = RNG.standard_normal((4, 16))
    pos = [0, 1, 777, 32767]
    got = oracle.rotate_f64(x, pos, oracle.rope_frequencies(16, 10000.0), pairing)
    for r in range(4):
        ref = _loop_rotate(list(x[r]), pos[r], 10000.0, pairing)
        assert np.max(np.abs(got[r] - np.array(ref))) <= 1e-12


def test_position_zero_is_identity():
    x = RNG.standard_normal((2, 3, 128))
    f = oracle.rope_frequencies(128, 500000.0)
    for pairing in ("half", "adjacent"):
        assert np.array_equal(oracle.rotate_f64(x, np.zeros((2, 3)), f, pairing), x)


def test_quarter_turn():
    # one pair, frequency pi/2, position 1: (a, b) -> (-b, a)
    x = np.array([[0.75, -2.5]])
    got = oracle.rotate_f64(x, [1], np.array([np.pi / 2]), "half")
    assert np.max(np.abs(got - np.array([[2.5, 0.75]]))) <= 1e-15


def test_pair_norms_preserved():
    x = RNG.standard_normal((6, 128)) * 3
    pos = RNG.integers(0, 1 << 20, size=6)
    y = oracle.rotate_f64(x, pos, oracle.rope_frequencies(128, 10000.0), "half")
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pairing", ["half", "adjacent"])
def test_scores_depend_on_relative_position_only(pairing):
    # <R(m) q, R(n) k> = <R(m + s) q, R(n + s) k> = <R(m - n) q, k>: the property
    # that makes rotated keys cacheable at their own positions
    D = 128
    f = oracle.model_frequencies(D, 500000.0, LLAMA3)
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    m, n = 9000, 1234
    base = np.dot(oracle.rotate_f64(q, m, f, pairing), oracle.rotate_f64(k, n, f, pairing))
    for s in (1, 517, 20000):
        sh = np.dot(oracle.rotate_f64(q, m + s, f, pairing), oracle.rotate_f64(k, n + s, f, pairing))
        assert abs(sh - base) <= 1e-9 * max(1.0, abs(base))
    rel = np.dot(oracle.rotate_f64(q, m - n, f, pairing), k)
    assert abs(rel - base) <= 1e-9 * max(1.0, abs(base))


# ------------------------------------------------------------ K/V write

def _step_case(B, T, Hq, Hkv, D, S, pos0, seed):
    q = workloads.bf16_randn((B, T, Hq, D), seed * 10 + 1)
    k = workloads.bf16_randn((B, T, Hkv, D), seed * 10 + 2)
    v = workloads.bf16_randn((B, T, Hkv, D), seed * 10 + 3)
    kc = workloads.bf16_randn((B, Hkv, S, D), seed * 10 + 4)
    vc = workloads.bf16_randn((B, Hkv, S, D), seed * 10 + 5)
    return q, k, v, np.asarray(pos0, dtype=np.int32), kc, vc


@pytest.mark.parametrize("pairing", ["half", "adjacent"])
def test_kv_write_slots_and_values(pairing):
    B, T, Hq, Hkv, D, S = 5, 4, 6, 2, 16, 40
    pos0 = [0, 17, 38, -3, 99]              # a row spilling past S_max, a negative and a large length
    q, k, v, p0, kc, vc = _step_case(B, T, Hq, Hkv, D, S, pos0, seed=7)
    qo, kco, vco = oracle.rope_kv_write(q, k, v, p0, kc, vc, theta=10000.0, pairing=pairing)
    f = oracle.rope_frequencies(D, 10000.0)
    expect_pos = {0: [0, 1, 2, 3], 1: [17, 18, 19, 20], 2: [38, 39, 40, 41], 3: [0, 1, 2, 3], 4: [40, 41, 42, 43]}
    written = np.zeros((B, S), dtype=bool)
    for b in range(B):
        for i, p in enumerate(expect_pos[b]):
            ref_q = _bits(_complex_rotate(_f64(q[b, i]), np.full(Hq, p), f, pairing))
            assert np.array_equal(qo[b, i], ref_q)
            if p >= S:
                continue
            written[b, p] = True
            ref_k = _bits(_complex_rotate(_f64(k[b, i]), np.full(Hkv, p), f, pairing))
            assert np.array_equal(kco[b, :, p], ref_k)
            assert np.array_equal(vco[b, :, p], v[b, i])
    # every other slot keeps its bytes
    keep = ~written[:, None, :, None]
    assert np.array_equal(np.where(keep, kco, 0), np.where(keep, kc, 0))
    assert np.array_equal(np.where(keep, vco, 0), np.where(keep, vc, 0))
    assert written.sum() == 4 + 4 + 2 + 4 + 0


def test_kv_write_at_position_zero_copies_k():
    q, k, v, p0, kc, vc = _step_case(2, 1, 4, 2, 64, 8, [0, 0], seed=8)
    qo, kco, vco = oracle.rope_kv_write(q, k, v, p0, kc, vc, theta=500000.0, llama3=LLAMA3)
    assert np.array_equal(qo, q)
    assert np.array_equal(kco[:, :, 0], k[:, 0])


def test_rotated_cache_attention_is_shift_invariant():
    # decode on a cache written by the step: shifting every position by s
    # (the whole prefix and the query) leaves the attention output unchanged
    D, Hq, Hkv, n = 64, 4, 2, 50
    f = oracle.rope_frequencies(D, 10000.0)
    qv = RNG.standard_normal((1, Hq, D))
    kv = RNG.standard_normal((1, Hkv, n, D))
    vv = RNG.standard_normal((1, Hkv, n, D))
    outs = []
    for s in (0, 1000):
        kr = oracle.rotate_f64(kv, (np.arange(n) + s)[None, None, :], f)
        qr = oracle.rotate_f64(qv, np.full((1, Hq), n - 1 + s), f)
        outs.append(oracle.decode_attention_f64(qr, kr, vv, [n], 0.125))
    assert np.max(np.abs(outs[0] - outs[1])) <= 1e-10


# ------------------------------------------------------- mutation tests

def _rope_battery(mod) -> list[str]:
    failed = []
    f = mod.rope_frequencies(32, 10000.0)

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:
            failed.append(name + "-raised")

    x = RNG.standard_normal((3, 32))
    pos = np.array([0, 5, 30000])
    check("complex-half", lambda: np.max(np.abs(mod.rotate_f64(x, pos, f, "half") - _complex_rotate(x, pos, f, "half"))) <= 1e-12)
    check("complex-adjacent", lambda: np.max(np.abs(mod.rotate_f64(x, pos, f, "adjacent") - _complex_rotate(x, pos, f, "adjacent"))) <= 1e-12)
    check("loops", lambda: np.max(np.abs(mod.rotate_f64(x[1], 5, f, "half") - np.array(_loop_rotate(list(x[1]), 5, 10000.0, "half")))) <= 1e-12)
    fr = mod.rope_frequencies(128, 500000.0)
    g = mod.llama3_scale_frequencies(fr, **LLAMA3)
    w = 2 * np.pi / fr
    check("llama3-keep", lambda: np.array_equal(g[w < 2048.0], fr[w < 2048.0]))
    check("llama3-slow", lambda: np.array_equal(g[w > 8192.0], fr[w > 8192.0] / 32.0))
    f_q = 2 * np.pi * 1.75 / 8192.0
    check("llama3-quarter", lambda: math.isclose(mod.llama3_scale_frequencies([f_q], 32.0, 1.0, 4.0, 8192.0)[0],
                                                 0.75 * f_q / 32.0 + 0.25 * f_q, rel_tol=1e-14))
    B, T, Hq, Hkv, D, S = 3, 3, 4, 2, 16, 12
    q, k, v, p0, kc, vc = _step_case(B, T, Hq, Hkv, D, S, [1, 10, -2], seed=9)

    def step_ok():
        qo, kco, vco = mod.rope_kv_write(q, k, v, p0, kc, vc, theta=10000.0)
        ff = mod.rope_frequencies(D, 10000.0)
        pos = {0: [1, 2, 3], 1: [10, 11, 12], 2: [0, 1, 2]}
        written = np.zeros((B, S), dtype=bool)
        for b in range(B):
            for i, p in enumerate(pos[b]):
                if not np.array_equal(qo[b, i], _bits(_complex_rotate(_f64(q[b, i]), np.full(Hq, p), ff, "half"))):
                    return False
                if p >= S:
                    continue
                written[b, p] = True
                if not np.array_equal(kco[b, :, p], _bits(_complex_rotate(_f64(k[b, i]), np.full(Hkv, p), ff, "half"))):
                    return False
                if not np.array_equal(vco[b, :, p], v[b, i]):
                    return False
        keep = ~written[:, None, :, None]
        return (np.array_equal(np.where(keep, kco, 0), np.where(keep, kc, 0))
                and np.array_equal(np.where(keep, vco, 0), np.where(keep, vc, 0)))
    check("step", step_ok)
    return failed


ROPE_MUTANTS = {
    "sin-sign": ("ra = a * c - b * s", "ra = a * c + b * s"),
    "half-pairs-adjacent": ("a, b = x[..., : D // 2], x[..., D // 2:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    "frequency-exponent": ("-(2.0 * j) / float(D)", "-(1.0 * j) / float(D)"),
    "position-off-by-one": ("p0[:, None] + np.arange(T", "p0[:, None] + 1 + np.arange(T"),
    "v-rotated": ("v_cache[b, kvh, p] = v_bits[b, i, kvh]", "v_cache[b, kvh, p] = k_rot[b, i, kvh]"),
    "k-written-one-slot-late": ("k_cache[b, kvh, p] = k_rot[b, i, kvh]", "k_cache[b, kvh, min(p + 1, S_max - 1)] = k_rot[b, i, kvh]"),
    "blend-weights-swapped": ("(1.0 - s) * f / float(factor) + s * f", "s * f / float(factor) + (1.0 - s) * f"),
    "high-region-flipped": ("if wavelen < high_wavelen:", "if wavelen > high_wavelen:"),
    "no-length-clamp": ("np.clip(np.asarray(pos0, dtype=np.int64), 0, S_max)", "np.asarray(pos0, dtype=np.int64)"),
    "slot-guard-off-by-one": ("if p >= S_max:", "if p > S_max:"),
}


def _load_rope_mutant(old: str, new: str) -> types.ModuleType:
    src = open(orope.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    src = src.replace("from .bf16 import f64_to_bf16_bits_rne", "from oracle.bf16 import f64_to_bf16_bits_rne")
    mod = types.ModuleType("rope_mutant")
    exec(compile(src, "rope_mutant", "exec"), mod.__dict__)
    return mod


def test_rope_battery_passes_on_oracle():
    assert _rope_battery(orope) == []


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_planted_rope_mistake_is_caught(name):
    old, new = ROPE_MUTANTS[name]
    with np.errstate(all="ignore"):
        failed = _rope_battery(_load_rope_mutant(old, new))
    assert failed, f"mutant {name} passed every pin"
