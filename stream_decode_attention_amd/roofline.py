"""Algorithmic byte counts and peaks for the roofline of decode attention.

Decode attention reads each attended key and value row once: for a call with
lengths n_b, the algorithmic traffic is sum_b n_b * Hkv * D * 2 (K and V) *
2 bytes (bf16). Query, output, lengths and the partial softmax state are
implementation overhead and are not counted. The roofline time is bytes over
bandwidth (llm-decode-cuda, roofline paragraph: bytes read per token over the
measured streaming bandwidth).
"""
from __future__ import annotations

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
BF16_BYTES = 2


def _clamp(n, s_max):
    return np.clip(np.asarray(n, dtype=np.int64), 0, s_max)


def kv_bytes_decode(lens, Hkv: int, D: int, S_max: int, elem_bytes: int = BF16_BYTES) -> int:
    """K and V bytes a decode call must read: sum_b clamp(n_b) * Hkv * D * 2 * elem_bytes."""
    return int(_clamp(lens, S_max).sum()) * Hkv * D * 2 * elem_bytes


def kv_bytes_chunk(ctx_lens, T: int, Hkv: int, D: int, S_max: int, elem_bytes: int = BF16_BYTES) -> int:
    """K and V bytes of a verify chunk read once for all T tokens: keys j < ctx + T."""
    return int(_clamp(np.asarray(ctx_lens, dtype=np.int64) + T, S_max).sum()) * Hkv * D * 2 * elem_bytes


def kv_bytes_per_token(layers: int, Hkv: int, D: int, elem_bytes: int) -> int:
    """KV-cache bytes one more token of context adds to every decode step."""
    return layers * Hkv * D * 2 * elem_bytes


def roofline_tokens_per_s(bandwidth_Bps: float, weight_bytes: float, ctx: int, kv_per_token: float) -> float:
    """Decode-step rate if the step only streams the weights and ctx tokens of KV cache."""
    return bandwidth_Bps / (weight_bytes + ctx * kv_per_token)


def partial_state_bytes(B: int, T: int, Hq: int, D: int, active_tiles_per_row) -> int:
    """Bytes of (m, l, acc) written for the active tiles (overhead, not algorithmic)."""
    return int(np.sum(active_tiles_per_row)) * (D + 2) * 4
