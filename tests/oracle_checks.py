"""Independent references used to pin the fp64 oracle.

Nothing here imports the oracle: each function restates the mathematics in a
different way (pure-Python loops with exact summation, or PyTorch's own
scaled_dot_product_attention in float64), so that agreement is evidence about
the oracle rather than a copy of it.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def brute_decode(q, k, v, lens, scale):
    """Pure-Python loops: q [B,Hq,D], k/v [B,Hkv,S,D] float arrays; math.fsum sums."""
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = min(max(int(lens[b]), 0), S)
        for h in range(Hq):
            if n == 0:
                continue
            kv = h // G
            s = [scale * math.fsum(float(q[b, h, d]) * float(k[b, kv, j, d]) for d in range(D))
                 for j in range(n)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            den = math.fsum(w)
            for d in range(D):
                out[b, h, d] = math.fsum(w[j] * float(v[b, kv, j, d]) for j in range(n)) / den
    return out


def sdpa_decode(q, k, v, lens, scale):
    """torch CPU scaled_dot_product_attention in float64, boolean mask j < n.

    K/V are expanded with repeat_interleave over the head axis, the copy that
    grouped-query index math avoids. Rows with n == 0 are set to zero.
    """
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    k = torch.as_tensor(np.asarray(k, dtype=np.float64))
    v = torch.as_tensor(np.asarray(v, dtype=np.float64))
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    n = torch.as_tensor(np.clip(np.asarray(lens), 0, S))
    mask = torch.arange(S)[None, :] < n[:, None]           # [B, S]
    mask = mask[:, None, None, :].expand(B, Hq, 1, S)
    safe = mask.clone()
    safe[..., 0] |= ~mask.any(-1)                         # keep empty rows finite
    o = torch.nn.functional.scaled_dot_product_attention(
        q[:, :, None, :], kk, vv, attn_mask=safe, scale=float(scale))[:, :, 0, :]
    o[~mask.any(-1)[..., 0]] = 0.0
    return o.numpy()


def sdpa_chunk(q, k, v, ctx, scale):
    """torch fp64 SDPA with an explicit causal mask: token i sees keys j < ctx + i + 1."""
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))  # [B, T, Hq, D]
    k = torch.as_tensor(np.asarray(k, dtype=np.float64))
    v = torch.as_tensor(np.asarray(v, dtype=np.float64))
    B, T, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    lim = torch.as_tensor(np.asarray(ctx))[:, None] + torch.arange(T)[None, :] + 1  # [B, T]
    lim = lim.clamp(0, S)
    mask = torch.arange(S)[None, None, :] < lim[:, :, None]                      # [B, T, S]
    mask = mask[:, None].expand(B, Hq, T, S)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), kk, vv, attn_mask=mask, scale=float(scale))
    return o.permute(0, 2, 1, 3).numpy()


def rand_f64(rng, *shape):
    return rng.standard_normal(shape)
