"""fp64 oracle for the step before attention: rotary position embedding of the
new tokens' q and k, and the write of their K/V into the static cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain NumPy in float64,
sharing nothing with the HIP library.

What the pages fix:
  * positions come from the device-resident lengths, and the K/V write is an
    indexed store at those positions; no shape depends on how far along the
    sequence is (tinydecode README, "how the decode step is put together");
  * q and k are rotated in place by a dedicated kernel (tinydecode README,
    "What's in here": in-place rope), fused with the K/V-cache write in
    llm-decode-cuda's engine (its per-layer step list puts the rotation and the
    cache write in one step);
  * the only rope scaling supported is the llama3 flavour (tinydecode README,
    "not done / known gaps").

Readings taken where the pages are silent (each restated where it is used):
  R1. Token i of row b (i < T) sits at position p = pos0[b] + i, where pos0 is
      the row's length before the step (seq_lens for decode, ctx_lens for a
      verify chunk). pos0 is clamped to [0, S_max] like every length; a token
      whose position is >= S_max has no cache slot: its K/V are not stored,
      and its q is still rotated at p.
  R2. The rotation is the textbook one (RoFormer): pair j of a head, j < D/2,
      turns by the angle p * f_j with f_j = theta^(-2j/D). Two pairings are
      in use and both are provided: "half" pairs (x_j, x_{j+D/2}) (the
      Hugging Face Llama layout, which tinydecode loads), "adjacent" pairs
      (x_{2j}, x_{2j+1}) (the RoFormer paper and Meta's reference code).
      A pair (a, b) becomes (a cos t - b sin t, a sin t + b cos t).
  R3. Angles are the exact real p * f_j (computed here in float64); no
      lower-precision frequency table is implied. Results are rounded once to
      the nearest-even bf16 (q out and the cached K); V is stored unchanged.
  R4. llama3 scaling (published with Llama 3.1): with wavelength
      w_j = 2 pi / f_j, L = original_max_position, frequencies whose
      wavelength is below L / high_freq_factor are kept, those above
      L / low_freq_factor are divided by `factor`, and in between the two are
      blended with weight s = (L / w_j - low_freq_factor) /
      (high_freq_factor - low_freq_factor) on the unscaled frequency.
"""
from __future__ import annotations

import numpy as np

from .bf16 import f64_to_bf16_bits_rne

PAIRINGS = ("half", "adjacent")


def _bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rope_frequencies(D: int, theta: float) -> np.ndarray:
    """f_j = theta^(-2j/D) for j < D/2 (reading R2), float64."""
    if D % 2:
        raise ValueError("D must be even")
    j = np.arange(D // 2, dtype=np.float64)
    return np.power(float(theta), -(2.0 * j) / float(D))


def llama3_scale_frequencies(freqs, factor: float, low_freq_factor: float,
                             high_freq_factor: float, original_max_position: float) -> np.ndarray:
    """The llama3 frequency scaling (reading R4), one frequency at a time."""
    L = float(original_max_position)
    low_wavelen = L / float(low_freq_factor)
    high_wavelen = L / float(high_freq_factor)
    out = []
    for f in np.asarray(freqs, dtype=np.float64):
        wavelen = 2.0 * np.pi / f
        if wavelen < high_wavelen:              # high frequencies: unchanged
            out.append(f)
        elif wavelen > low_wavelen:             # low frequencies: slowed by `factor`
            out.append(f / float(factor))
        else:                                   # in between: blend of the two
            s = (L / wavelen - float(low_freq_factor)) / (float(high_freq_factor) - float(low_freq_factor))
            out.append((1.0 - s) * f / float(factor) + s * f)
    return np.asarray(out, dtype=np.float64)


def model_frequencies(D: int, theta: float, llama3: dict | None = None) -> np.ndarray:
    """Frequencies of a model: plain (R2), or llama3-scaled (R4) when `llama3`
    holds factor, low_freq_factor, high_freq_factor, original_max_position."""
    f = rope_frequencies(D, theta)
    if llama3:
        f = llama3_scale_frequencies(f, llama3["factor"], llama3["low_freq_factor"],
                                     llama3["high_freq_factor"], llama3["original_max_position"])
    return f


def rotate_f64(x, positions, freqs, pairing: str = "half") -> np.ndarray:
    """Rotate the last axis (D) of x by position (reading R2), float64.

    x: [..., D]; positions: broadcastable to x.shape[:-1]; freqs: [D/2].
    """
    if pairing not in PAIRINGS:
        raise ValueError(f"pairing must be one of {PAIRINGS}")
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    freqs = np.asarray(freqs, dtype=np.float64)
    assert freqs.shape == (D // 2,)
    pos = np.asarray(positions, dtype=np.float64)[..., None]
    ang = pos * freqs                                   # [..., D/2]
    c, s = np.cos(ang), np.sin(ang)
    if pairing == "half":
        a, b = x[..., : D // 2], x[..., D // 2:]
    else:
        a, b = x[..., 0::2], x[..., 1::2]
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty_like(x)
    if pairing == "half":
        out[..., : D // 2], out[..., D // 2:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out


def token_positions(pos0, T: int, S_max: int) -> np.ndarray:
    """[B, T] positions pos0[b] + i with pos0 clamped to [0, S_max] (reading R1)."""
    p0 = np.clip(np.asarray(pos0, dtype=np.int64), 0, S_max)
    return p0[:, None] + np.arange(T, dtype=np.int64)[None, :]


def rope_kv_write_f64(q, k_new, positions, freqs, pairing: str = "half"):
    """Rotated q [B,T,Hq,D] and k [B,T,Hkv,D] in float64 (no rounding)."""
    pos = np.asarray(positions)[:, :, None]             # broadcast over heads
    return rotate_f64(q, pos, freqs, pairing), rotate_f64(k_new, pos, freqs, pairing)


def rope_kv_write(q_bits, k_bits, v_bits, pos0, k_cache_bits, v_cache_bits, *, theta: float,
                  pairing: str = "half", llama3: dict | None = None):
    """The whole step on bf16 bit patterns (readings R1-R4).

    q_bits [B,T,Hq,D], k_bits / v_bits [B,T,Hkv,D]: the new tokens' vectors;
    pos0 [B]: each row's length before the step; k_cache_bits / v_cache_bits
    [B,Hkv,S_max,D]: the caches before the step (not modified).
    Returns (q_out_bits, k_cache_out_bits, v_cache_out_bits).
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    B, T, Hq, D = q_bits.shape
    Hkv = k_bits.shape[2]
    S_max = k_cache_bits.shape[2]
    assert k_bits.shape == v_bits.shape == (B, T, Hkv, D)
    assert k_cache_bits.shape == v_cache_bits.shape == (B, Hkv, S_max, D)
    freqs = model_frequencies(D, theta, llama3)
    positions = token_positions(pos0, T, S_max)
    qr, kr = rope_kv_write_f64(_bits_to_f64(q_bits), _bits_to_f64(k_bits), positions, freqs, pairing)
    q_out = f64_to_bf16_bits_rne(qr)
    k_rot = f64_to_bf16_bits_rne(kr)
    k_cache = np.array(k_cache_bits, dtype=np.uint16, copy=True)
    v_cache = np.array(v_cache_bits, dtype=np.uint16, copy=True)
    for b in range(B):
        for i in range(T):
            p = int(positions[b, i])
            if p >= S_max:                              # no slot (reading R1)
                continue
            for kvh in range(Hkv):
                k_cache[b, kvh, p] = k_rot[b, i, kvh]
                v_cache[b, kvh, p] = v_bits[b, i, kvh]
    return q_out, k_cache, v_cache
