"""Decode and chunk attention, written out in float64 (test infrastructure only).

What is computed (tinydecode README, "how the decode step is put together"):
the query of head h attends keys j < seq_len of its batch row; a query head maps
to a kv head in index math (grouped-query attention, no copies). For one query
vector q and the first n cached keys/values,

    s_j   = scale * <q, k_j>,            j = 0 .. n-1
    out   = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)

Readings taken where the pages are silent:

* kv head of query head h is h // G with G = Hq / Hkv (contiguous groups: the
  layout that repeat_interleave over the head axis would give);
* seq_len counts keys already in the cache, so keys j in [0, seq_len) are
  attended (the current token's K/V is written before attention);
* seq_len is clamped to [0, S_max]; an empty row (n = 0) outputs zeros;
* ``scale`` is the fp32 value handed to the kernel, widened exactly to fp64;
* chunk/verify query token i of a sequence with context ctx attends keys
  j < ctx + i + 1 (tinydecode README, "speculative decoding": the verify pass
  runs k+1 tokens on top of the existing context).

parity unpinned: none — every function here is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the top half of an IEEE binary32; shifting the 16 bits up
    gives that binary32 exactly, and binary32 -> binary64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Grouped-query mapping: query head h reads kv head h // (Hq / Hkv)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _clamp_len(n, S_max: int) -> int:
    return int(min(max(int(n), 0), S_max))


def _softmax_weighted_sum(scores: np.ndarray, V: np.ndarray) -> np.ndarray:
    """sum_j softmax(scores)_j * V[j], with the maximum subtracted first."""
    w = np.exp(scores - scores.max())
    return (w @ V) / w.sum()


def decode_attention_f64(q, k, v, seq_lens, scale, rows=None) -> np.ndarray:
    """Single-query decode attention over float64 arrays.

    q [B, Hq, D]; k, v [B, Hkv, S_max, D]; seq_lens [B]; returns [B, Hq, D].
    ``rows`` optionally restricts the work to a list of (b, h) pairs (other
    outputs stay zero), so full-size workloads can be sampled row by row.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, S_max = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    want = None if rows is None else set((int(b), int(h)) for b, h in rows)
    for b in range(B):
        n = _clamp_len(seq_lens[b], S_max)
        if n == 0:
            continue
        for h in range(Hq):
            if want is not None and (b, h) not in want:
                continue
            kvh = kv_head_of(h, Hq, Hkv)
            K = np.asarray(k[b, kvh, :n], dtype=np.float64)
            V = np.asarray(v[b, kvh, :n], dtype=np.float64)
            s = float(scale) * (K @ q[b, h])
            out[b, h] = _softmax_weighted_sum(s, V)
    return out


def decode_attention(q_bits, k_bits, v_bits, seq_lens, scale, rows=None) -> np.ndarray:
    """decode_attention_f64 on bf16 bit arrays (the bytes the GPU receives).

    Only the cache rows actually attended are widened, one (batch, kv head)
    slice at a time, which keeps the 32k-context workload within memory.
    """
    q = bf16_bits_to_f64(q_bits)
    B, Hq, D = q.shape
    Hkv, S_max = k_bits.shape[1], k_bits.shape[2]
    G = Hq // Hkv
    scale = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    want = None if rows is None else set((int(b), int(h)) for b, h in rows)
    for b in range(B):
        n = _clamp_len(seq_lens[b], S_max)
        if n == 0:
            continue
        for kvh in range(Hkv):
            heads = [h for h in range(kvh * G, kvh * G + G)
                     if want is None or (b, h) in want]
            if not heads:
                continue
            K = bf16_bits_to_f64(k_bits[b, kvh, :n])
            V = bf16_bits_to_f64(v_bits[b, kvh, :n])
            for h in heads:
                assert kv_head_of(h, Hq, Hkv) == kvh
                s = scale * (K @ q[b, h])
                out[b, h] = _softmax_weighted_sum(s, V)
    return out


def _chunk_one_sequence(q, K, V, ctx: int, S_max: int, scale: float) -> np.ndarray:
    """Verify attention for one sequence.

    q [T, Hq, D] float64; K, V [Hkv, span, D] float64 holding at least the
    attended keys (span >= min(ctx + T, S_max)). The mask is an explicit boolean
    matrix over keys j < ctx + T, applied to the whole score matrix, rather than
    a per-row slice, so that comparing against single-query decode calls checks
    the mask instead of running the same code twice.
    """
    T, Hq, D = q.shape
    Hkv = K.shape[0]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    limits = np.array([_clamp_len(ctx + i + 1, S_max) for i in range(T)])
    span = int(limits.max())
    if span == 0:
        return out
    j = np.arange(span)
    mask = j[None, :] < limits[:, None]                  # [T, span]
    for h in range(Hq):
        kvh = kv_head_of(h, Hq, Hkv)
        Kh, Vh = K[kvh, :span], V[kvh, :span]
        S = scale * (q[:, h, :] @ Kh.T)                  # [T, span]
        S = np.where(mask, S, -np.inf)
        for i in range(T):
            if limits[i] == 0:
                continue
            out[i, h] = _softmax_weighted_sum(S[i], Vh)
    return out


def chunk_attention_f64(q, k, v, ctx_lens, scale) -> np.ndarray:
    """Causal multi-query ("chunk") attention for speculative verification.

    q [B, T, Hq, D]; k, v [B, Hkv, S_max, D]; ctx_lens [B]; returns [B, T, Hq, D].
    Query token i attends keys j < ctx + i + 1: its own key is included, the T
    tokens' K/V sitting at positions ctx .. ctx+T-1 (tinydecode README,
    "speculative decoding": the verify pass is attention over k+1 tokens on top
    of the existing context).
    """
    q = np.asarray(q, dtype=np.float64)
    S_max = k.shape[2]
    return np.stack([
        _chunk_one_sequence(q[b], np.asarray(k[b], dtype=np.float64),
                            np.asarray(v[b], dtype=np.float64),
                            int(ctx_lens[b]), S_max, float(scale))
        for b in range(q.shape[0])])


def chunk_attention(q_bits, k_bits, v_bits, ctx_lens, scale) -> np.ndarray:
    """chunk_attention_f64 on bf16 bit arrays; only the attended span is widened."""
    q = bf16_bits_to_f64(q_bits)
    T = q.shape[1]
    S_max = k_bits.shape[2]
    scale = float(np.float32(scale))
    outs = []
    for b in range(q.shape[0]):
        ctx = int(ctx_lens[b])
        span = _clamp_len(ctx + T, S_max)
        K = bf16_bits_to_f64(k_bits[b, :, :span])
        V = bf16_bits_to_f64(v_bits[b, :, :span])
        outs.append(_chunk_one_sequence(q[b], K, V, ctx, S_max, scale))
    return np.stack(outs)


def split_kv_attention_f64(q, k, v, seq_lens, scale, chunk: int) -> np.ndarray:
    """Split-KV ("flash-decoding") form of decode_attention_f64.

    tinydecode README, "how the decode step is put together": each tile of
    ``chunk`` keys yields partial softmax state (m, l, acc) -- the tile's score
    maximum, the sum of exp(s - m) and the unnormalised sum of exp(s - m) v --
    and a second step merges the tiles with the log-sum-exp rule
    (llm-decode-cuda, attention section):

        M = max_c m_c,  w_c = exp(m_c - M),
        out = sum_c w_c acc_c / sum_c w_c l_c.

    Only tiles holding at least one key j < n exist. Used by the tests to pin
    the merge arithmetic against the flat definition.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, S_max = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = _clamp_len(seq_lens[b], S_max)
        n_tiles = -(-n // chunk)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            ms, ls, accs = [], [], []
            for c in range(n_tiles):
                lo, hi = c * chunk, min((c + 1) * chunk, n)
                K = np.asarray(k[b, kvh, lo:hi], dtype=np.float64)
                V = np.asarray(v[b, kvh, lo:hi], dtype=np.float64)
                s = float(scale) * (K @ q[b, h])
                m = s.max()
                p = np.exp(s - m)
                ms.append(m)
                ls.append(p.sum())
                accs.append(p @ V)
            if not ms:
                continue
            M = max(ms)
            w = np.exp(np.array(ms) - M)
            L = float(np.dot(w, ls))
            out[b, h] = (w @ np.array(accs)) / L
    return out
