"""fp64 oracle for the weight products of a decode step (matrix times a few
activation vectors), with bf16 or INT8 weight-only weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain NumPy, sharing
nothing with the HIP library.

What the pages fix (llm-decode-cuda, roofline paragraph and GEMV table, and
the INT8 section):
  * a decode step multiplies each activation vector by every weight matrix;
    weights are row-major [out][in], each read once per step, so the product
    is bound by the bytes read;
  * INT8 weight-only: the codes are symmetric and scaled per output row (one
    fp32 factor per row), computed once at load time, and widened back to
    real values inside the product;
  * a batch of sequences reads the weights once per step.

Readings taken where the pages are silent (restated where used):
  G1. y[b, n] = sum_k W[n, k] x[b, k]: W [N][K] row-major, x [B][K], y [B][N].
      Inputs are bf16 (this library's cache and activation type; the pages'
      engine uses fp16), the sum is exact here (fp64) and fp32 on the GPU.
  G2. Quantization of row n, in fp32 (the precision of the stored scale, so
      that both sides take the same integer decisions): a = max_k |W[n, k]|,
      s = a / 127 (one fp32 division), q = round_half_even(W[n, k] / s)
      (one fp32 division per weight), kept in [-127, 127]; a row of zeros
      gets s = 0 and q = 0.
  G3. The INT8 product is y[b, n] = s[n] * sum_k q[n, k] x[b, k].
"""
from __future__ import annotations

import numpy as np

Q_MAX = 127


def _bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gemv_f64(W, x) -> np.ndarray:
    """y = x W^T in float64 (reading G1); W [N][K], x [B][K] -> y [B][N]."""
    W = np.asarray(W, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return x @ W.T


def gemv(W_bits, x_bits) -> np.ndarray:
    """gemv_f64 on bf16 bit arrays (exact widening)."""
    return gemv_f64(_bits_to_f32(W_bits), _bits_to_f32(x_bits))


def quantize_rows_int8(W_bits):
    """Per-output-row symmetric INT8 quantization in fp32 (reading G2).

    Returns (q int8 [N][K], s float32 [N]).
    """
    W = _bits_to_f32(W_bits)                                  # exact
    N, K = W.shape
    q = np.zeros((N, K), dtype=np.int8)
    s = np.zeros(N, dtype=np.float32)
    for n in range(N):
        a = np.float32(np.max(np.abs(W[n]))) if K else np.float32(0)
        if a == 0:
            continue
        sn = np.float32(a / np.float32(Q_MAX))                # one fp32 division
        r = np.rint((W[n] / sn).astype(np.float32))           # fp32 division, ties to even
        q[n] = np.clip(r, -Q_MAX, Q_MAX).astype(np.int8)
        s[n] = sn
    return q, s


def gemv_int8_f64(q, s, x) -> np.ndarray:
    """y[b, n] = s[n] * sum_k q[n, k] x[b, k] in float64 (reading G3)."""
    qd = np.asarray(q, dtype=np.float64)
    sd = np.asarray(s, dtype=np.float64)
    return sd[None, :] * (np.asarray(x, dtype=np.float64) @ qd.T)


def gemv_int8(q, s, x_bits) -> np.ndarray:
    """gemv_int8_f64 with bf16 activations given as bit arrays."""
    return gemv_int8_f64(q, s, _bits_to_f32(x_bits))
