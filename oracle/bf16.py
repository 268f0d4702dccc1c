"""bf16 rounding of float64 results (test infrastructure only).

bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits and 7
fraction bits. These helpers find, for a float64 value, the two adjacent bf16
values around it and the round-to-nearest-even choice between them, working on
exact float64 comparisons rather than on a chain of conversions (which could
round twice).
"""
from __future__ import annotations

import numpy as np


def _bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers that increase with the value (-0 and +0 collide)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _from_ordered(o: np.ndarray) -> np.ndarray:
    o = np.asarray(o, dtype=np.int64)
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def bf16_bracket(x) -> tuple[np.ndarray, np.ndarray]:
    """(lo, hi): the largest bf16 <= x and the smallest bf16 >= x, as bit patterns.

    For x exactly representable in bf16, lo == hi. Values beyond the finite
    bf16 range are not supported (they never occur in the attention outputs).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_bracket needs finite inputs")
    # a starting guess within one bf16 step of x: the binary32 nearest x,
    # with its low 16 bits dropped
    guess = (x.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    o = _ordered(guess)
    cands = [o - 2, o - 1, o, o + 1, o + 2]
    vals = [_bits_to_f64(_from_ordered(c)) for c in cands]
    lo = np.full(x.shape, np.iinfo(np.int64).min, dtype=np.int64)
    hi = np.full(x.shape, np.iinfo(np.int64).max, dtype=np.int64)
    for c, v in zip(cands, vals):
        lo = np.where((v <= x) & (c > lo), c, lo)
        hi = np.where((v >= x) & (c < hi), c, hi)
    return _from_ordered(lo), _from_ordered(hi)


def f64_to_bf16_bits_rne(x) -> np.ndarray:
    """Round float64 to the nearest bf16, ties to the even fraction pattern."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = bf16_bracket(x)
    vlo, vhi = _bits_to_f64(lo), _bits_to_f64(hi)
    dlo, dhi = x - vlo, vhi - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0) & (lo != hi))
    out = np.where(pick_hi, hi, lo).astype(np.uint16)
    # keep the sign of zero results
    zero = (x == 0)
    return np.where(zero, np.where(np.signbit(x), 0x8000, 0).astype(np.uint16), out)
