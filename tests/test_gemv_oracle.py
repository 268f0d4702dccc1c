"""Pins for the GEMV / INT8 weight-only oracle (CPU only).

The pages give no numeric GEMV example, so the oracle is pinned by brute
force (scalar loops with math.fsum for the products, scalar np.float32
arithmetic for the quantizer), closed forms (identity and permutation
matrices, a hand-worked quantized row), invariants (power-of-two scaling,
negation, batch-row independence, the half-step rounding bound, zero rows),
and mutation tests: plausible mistakes planted in a copy of the oracle must
each fail one of these pins.
"""
from __future__ import annotations

import importlib
import math
import types

import numpy as np
import pytest

import oracle
ogemv = importlib.import_module("oracle.gemv")     # the module (oracle.gemv is also a function name)
import workloads

RNG = np.random.default_rng(20261204)


def _f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bits(values):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    v = np.asarray(values, dtype=np.float32)
    b = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(_f32(b), v), "test values must be exact in bf16"
    return b


def _brute_gemv(W, x):
    N, K = W.shape
    return np.array([[math.fsum(float(W[n, k]) * float(x[b, k]) for k in range(K)) for n in range(N)]
                     for b in range(x.shape[0])])


def _brute_quantize_row(w):
    """Scalar np.float32 arithmetic, one element at a time."""
    a = np.float32(0)
    for v in w:
        a = max(a, np.float32(abs(v)))
    if a == 0:
        return [0] * len(w), np.float32(0)
    s = np.float32(a) / np.float32(127)
    q = []
    for v in w:
        t = np.float32(v) / s
        r = int(np.rint(t))
        q.append(max(-127, min(127, r)))
    return q, np.float32(s)


# ------------------------------------------------------------------ GEMV

@pytest.mark.parametrize("B,N,K", [(1, 3, 5), (2, 7, 16), (4, 5, 33)])
def test_gemv_matches_brute_force(B, N, K):
    W = workloads.bf16_randn((N, K), 11 * N + K)
    x = workloads.bf16_randn((B, K), 13 * B + K)
    got = oracle.gemv(W, x)
    ref = _brute_gemv(_f32(W), _f32(x))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_gemv_identity_and_permutation():
    K = 24
    x = workloads.bf16_randn((3, K), 5)
    eye = _bits(np.eye(K))
    assert np.array_equal(oracle.gemv(eye, x), _f32(x).astype(np.float64))
    perm = RNG.permutation(K)
    P = _bits(np.eye(K)[perm])
    assert np.array_equal(oracle.gemv(P, x), _f32(x).astype(np.float64)[:, perm])


def test_gemv_rows_of_x_are_independent():
    W = workloads.bf16_randn((9, 40), 6)
    x = workloads.bf16_randn((4, 40), 7)
    full = oracle.gemv(W, x)
    for b in range(4):
        assert np.array_equal(oracle.gemv(W, x[b:b + 1])[0], full[b])


# --------------------------------------------------------- quantization

def test_quantize_hand_worked_row():
    # a = 1, s = fl32(1/127); 0.5/s and 0.25/s land clear of ties (63.5000, 31.75)
    q, s = oracle.quantize_rows_int8(_bits([[0.5, -1.0, 0.25, 0.0]]))
    assert s[0] == np.float32(1.0) / np.float32(127)
    assert q.tolist() == [[64, -127, 32, 0]]


def test_quantize_matches_scalar_brute_force():
    W = workloads.bf16_randn((6, 37), 8)
    q, s = oracle.quantize_rows_int8(W)
    Wf = _f32(W)
    for n in range(6):
        bq, bs = _brute_quantize_row(Wf[n])
        assert q[n].tolist() == bq and s[n] == bs


def test_quantize_invariants():
    W = workloads.bf16_randn((16, 256), 9)
    q, s = oracle.quantize_rows_int8(W)
    Wf = _f32(W).astype(np.float64)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(np.int32)) <= 127)
    # the largest magnitude of each row maps to +-127
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    # rounding: within half a step, plus the fp32 rounding of the quotient
    # w / s (at most 127 * 2^-24 steps)
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - Wf)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # negation flips every code, keeps the scale
    qn, sn = oracle.quantize_rows_int8(W ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # scaling by a power of two is exact in bf16 and fp32: same codes, scale x4
    W4 = workloads.bf16_scale(W, np.ones(W.shape[:-1] + (1,), bool), 4.0)
    q4, s4 = oracle.quantize_rows_int8(W4)
    assert np.array_equal(q4, q) and np.array_equal(s4, s * np.float32(4))


def test_quantize_zero_row():
    W = workloads.bf16_randn((3, 16), 10)
    W[1] = 0
    q, s = oracle.quantize_rows_int8(W)
    assert s[1] == 0 and np.all(q[1] == 0)


def test_int8_gemv_equals_float_gemv_on_dequantized_weights():
    W = workloads.bf16_randn((12, 64), 11)
    x = workloads.bf16_randn((3, 64), 12)
    q, s = oracle.quantize_rows_int8(W)
    deq = q.astype(np.float64) * s[:, None].astype(np.float64)
    assert np.max(np.abs(oracle.gemv_int8(q, s, x) - oracle.gemv_f64(deq, _f32(x)))) <= 1e-12
    # and it is close to the unquantized product: at most half a step per weight
    bound = 0.5 * s[None, :] * np.abs(_f32(x)).astype(np.float64).sum(1)[:, None] * 1.000001
    assert np.all(np.abs(oracle.gemv_int8(q, s, x) - oracle.gemv(W, x)) <= bound)


# ------------------------------------------------------- mutation tests

def _gemv_battery(mod) -> list[str]:
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:
            failed.append(name + "-raised")

    W = workloads.bf16_randn((8, 8), 21)
    x = workloads.bf16_randn((2, 8), 22)
    check("brute", lambda: np.max(np.abs(mod.gemv(W, x) - _brute_gemv(_f32(W), _f32(x)))) <= 1e-12)
    check("hand", lambda: mod.quantize_rows_int8(_bits([[0.5, -1.0, 0.25, 0.0]]))[0].tolist() == [[64, -127, 32, 0]])

    def scalar():
        Wq = workloads.bf16_randn((4, 19), 23)
        q, s = mod.quantize_rows_int8(Wq)
        for n in range(4):
            bq, bs = _brute_quantize_row(_f32(Wq)[n])
            if q[n].tolist() != bq or s[n] != bs:
                return False
        return True
    check("scalar-quantize", scalar)

    def zero_row():
        Wz = workloads.bf16_randn((2, 8), 24)
        Wz[0] = 0
        q, s = mod.quantize_rows_int8(Wz)
        return s[0] == 0 and np.all(q[0] == 0)
    check("zero-row", zero_row)

    def int8_product():
        Wi = workloads.bf16_randn((6, 16), 25)
        xi = workloads.bf16_randn((2, 16), 26)
        q, s = oracle.quantize_rows_int8(Wi)             # the reference codes
        deq = q.astype(np.float64) * s[:, None].astype(np.float64)
        return np.max(np.abs(mod.gemv_int8(q, s, xi) - _brute_gemv(deq, _f32(xi)))) <= 1e-12
    check("int8-product", int8_product)
    return failed


GEMV_MUTANTS = {
    "transposed-weights": ("return x @ W.T\n", "return x @ W\n"),
    "scale-dropped": ("return sd[None, :] * (np.asarray(x, dtype=np.float64) @ qd.T)",
                      "return (np.asarray(x, dtype=np.float64) @ qd.T)"),
    "scale-per-column": ("return sd[None, :] * (np.asarray(x, dtype=np.float64) @ qd.T)",
                         "return (np.asarray(x, dtype=np.float64) * sd[None, :qd.shape[1]]) @ qd.T"),
    "divide-by-128": ("sn = np.float32(a / np.float32(Q_MAX))", "sn = np.float32(a / np.float32(128))"),
    "floor-rounding": ("r = np.rint((W[n] / sn).astype(np.float32))", "r = np.floor((W[n] / sn).astype(np.float32))"),
    "max-not-abs": ("a = np.float32(np.max(np.abs(W[n]))) if K else np.float32(0)",
                    "a = np.float32(np.max(W[n])) if K else np.float32(0)"),
}


def _load_gemv_mutant(old, new):
    src = open(ogemv.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("gemv_mutant")
    exec(compile(src.replace(old, new, 1), "gemv_mutant", "exec"), mod.__dict__)
    return mod


def test_gemv_battery_passes_on_oracle():
    assert _gemv_battery(ogemv) == []


@pytest.mark.parametrize("name", sorted(GEMV_MUTANTS))
def test_planted_gemv_mistake_is_caught(name):
    old, new = GEMV_MUTANTS[name]
    with np.errstate(all="ignore"):
        failed = _gemv_battery(_load_gemv_mutant(old, new))
    assert failed, f"mutant {name} passed every pin"
