"""Seeded synthetic inputs for split-KV decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the fp64 oracle (through the tests) and the HIP path
consume exactly the bytes produced here.

Shapes follow the models the pages measure or name:

* SmolLM2-360M (15 query heads, 5 kv heads, head dim 64, 32 layers): the model
  of the llm-decode-cuda write-up, whose KV cache is laid out per layer as
  [sequence][kv_head][position][64] (design notes of that page).
* TinyLlama-1.1B (32/4 heads, dim 64, 22 layers) and Llama-3 shapes: the models
  tinydecode loads (tinydecode README, "using it").
* Llama-3.2-3B (24/8 heads, dim 128) for the speculative verify chunk of k+1
  query tokens (tinydecode README, "speculative decoding").

The pages measure whole models on real text; here every tensor is bf16 drawn
from N(0, 1) (float32 normal samples from NumPy's PCG64, rounded to
nearest-even bf16), which stands in for real activations. Cache slots at or
past a sequence's length hold random data too, unless a test overwrites them.

Seeds: seed = 100000*cfg + 10*layer + t with t = 1 (q), 2 (K), 3 (V),
4 (outlier mask), 5 (lengths).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "bf16_randn", "make_case", "make_config",
    "seed_for", "bf16_scale", "uniform_mask", "ragged_lens", "BF16_NAN",
    "SPEC_VOCABS", "spec_sampling_case", "spec_greedy_case",
]

# A quiet-NaN bf16 pattern, used by tests to poison cache slots that must never be read.
BF16_NAN = 0x7FC0

T_Q, T_K, T_V, T_OUTLIER, T_LENS = 1, 2, 3, 4, 5


def seed_for(cfg: int, layer: int, t: int) -> int:
    return 100000 * cfg + 10 * layer + t


_BLOCK = 1 << 20          # elements per independently seeded block


def _round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of finite float32 samples."""
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def _fill_blocks(n: int, seed: int, make_block, dtype) -> np.ndarray:
    """Run make_block(rng, count) over fixed 1 Mi-element blocks, block i drawing
    from its own child of SeedSequence(seed); the bytes do not depend on the
    number of worker threads."""
    out = np.empty(n, dtype=dtype)
    nblk = -(-n // _BLOCK)
    children = np.random.SeedSequence(int(seed)).spawn(nblk)

    def work(i):
        lo, hi = i * _BLOCK, min((i + 1) * _BLOCK, n)
        out[lo:hi] = make_block(np.random.default_rng(children[i]), hi - lo)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(work, range(nblk)))
    return out


def _normal_block(rng, count):
    return _round_to_bf16_bits(rng.standard_normal(count, dtype=np.float32))


def bf16_randn(shape, seed: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) samples: float32 normals from NumPy's
    PCG64, rounded to nearest-even bf16."""
    n = int(np.prod(shape))
    return _fill_blocks(n, seed, _normal_block, np.uint16).reshape(shape)


def uniform_mask(shape, frac: float, seed: int) -> np.ndarray:
    """Boolean mask with each entry True with probability ``frac``."""
    n = int(np.prod(shape))
    return _fill_blocks(n, seed, lambda rng, k: rng.random(k) < frac, np.bool_).reshape(shape)


def bf16_scale(x_bits: np.ndarray, mask: np.ndarray, factor: float) -> np.ndarray:
    """Multiply the bf16 values selected by ``mask`` (broadcast over the last
    axis) by ``factor``, a power of two, which is exact in bf16."""
    e = int(round(np.log2(factor)))
    assert 2.0 ** e == factor, "factor must be a power of two"
    out = x_bits.copy()
    sel = np.broadcast_to(mask, x_bits.shape)
    bits = out[sel].astype(np.int32)
    exp = (bits >> 7) & 0xFF
    nz = exp != 0                     # zeros and subnormals never occur in N(0,1) bf16 draws
    bits[nz] += e << 7
    out[sel] = bits.astype(np.uint16)
    return out


@dataclass(frozen=True)
class Workload:
    """One of the five measured shapes."""
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S_max: int
    lens: tuple            # candidate lengths (decode) or context lengths (chunk)
    layers: int = 1
    T: int = 1             # query tokens per sequence (chunk/verify when > 1)
    chunk: int = 0         # keys per split tile; 0 = library default
    outlier_frac: float = 0.0
    outlier_factor: float = 8.0
    ragged: bool = False   # lengths drawn per sequence from U[1, S_max]
    notes: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        # the softmax scale travels through the C ABI as fp32
        return float(np.float32(1.0 / math.sqrt(self.D)))


CONFIGS = {
    1: Workload(1, "smollm2-360m-single-call", B=1, Hq=15, Hkv=5, D=64, S_max=128,
                lens=(64,), chunk=32,
                notes="one call, fp32 and bf16 output"),
    2: Workload(2, "smollm2-360m-32-layer-decode", B=1, Hq=15, Hkv=5, D=64, S_max=4096,
                lens=(64, 1024, 2048, 4096), layers=32,
                notes="32 independent calls per step, one graph replay"),
    3: Workload(3, "tinyllama-1.1b-22-layer-decode", B=1, Hq=32, Hkv=4, D=64, S_max=8192,
                lens=(1024, 4096, 8192), layers=22, outlier_frac=0.05,
                notes="5% of keys scaled x8"),
    4: Workload(4, "llama3-8b-batched-ragged-decode", B=8, Hq=32, Hkv=8, D=128, S_max=32768,
                lens=(), ragged=True,
                notes="seq_lens ~ U[1, 32768] per sequence"),
    5: Workload(5, "llama3.2-3b-verify-chunk", B=1, Hq=24, Hkv=8, D=128, S_max=16384,
                lens=(8192,), T=6,
                notes="T = k+1 = 6 query tokens on 8192 keys of context"),
}


def make_case(B, Hq, Hkv, D, S_max, lens, *, T=1, seed=0, outlier_frac=0.0,
              outlier_factor=8.0):
    """Random bf16 q/K/V for arbitrary shapes.

    Returns a dict with bf16 bit arrays ``q`` ([B,Hq,D] when T == 1, else
    [B,T,Hq,D]), ``k`` and ``v`` ([B,Hkv,S_max,D]), int32 ``lens`` [B] and the
    fp32 ``scale`` 1/sqrt(D).
    """
    qshape = (B, Hq, D) if T == 1 else (B, T, Hq, D)
    q = bf16_randn(qshape, seed * 10 + T_Q)
    k = bf16_randn((B, Hkv, S_max, D), seed * 10 + T_K)
    v = bf16_randn((B, Hkv, S_max, D), seed * 10 + T_V)
    if outlier_frac > 0:
        mask = uniform_mask((B, Hkv, S_max), outlier_frac, seed * 10 + T_OUTLIER)
        k = bf16_scale(k, mask[..., None], outlier_factor)
    lens = np.asarray(lens, dtype=np.int32).reshape(B)
    return {"q": q, "k": k, "v": v, "lens": lens,
            "scale": float(np.float32(1.0 / math.sqrt(D)))}


def ragged_lens(cfg: int, B: int, S_max: int, layer: int = 0) -> np.ndarray:
    """Per-sequence lengths drawn uniformly from [1, S_max]."""
    rng = np.random.default_rng(seed_for(cfg, layer, T_LENS))
    return rng.integers(1, S_max + 1, size=B).astype(np.int32)


def make_config(cfg: int, layer: int = 0, n: int | None = None) -> dict:
    """Inputs of workload ``cfg`` for one layer.

    ``n`` picks the sequence (decode) or context (chunk) length; by default the
    largest listed length, or ragged per-sequence lengths for workload 4.
    """
    w = CONFIGS[cfg]
    qshape = (w.B, w.Hq, w.D) if w.T == 1 else (w.B, w.T, w.Hq, w.D)
    q = bf16_randn(qshape, seed_for(cfg, layer, T_Q))
    k = bf16_randn((w.B, w.Hkv, w.S_max, w.D), seed_for(cfg, layer, T_K))
    v = bf16_randn((w.B, w.Hkv, w.S_max, w.D), seed_for(cfg, layer, T_V))
    if w.outlier_frac > 0:
        mask = uniform_mask((w.B, w.Hkv, w.S_max), w.outlier_frac, seed_for(cfg, layer, T_OUTLIER))
        k = bf16_scale(k, mask[..., None], w.outlier_factor)
    if w.ragged:
        lens = ragged_lens(cfg, w.B, w.S_max, layer)
    else:
        lens = np.full((w.B,), max(w.lens) if n is None else n, dtype=np.int32)
    return {"q": q, "k": k, "v": v, "lens": lens, "scale": w.scale, "workload": w}


# ---------------------------------------------------------------------------
# Inputs of the speculative accept/reject step.
#
# The verify pass of the pages' speculative loops scores k + 1 positions of
# a target model: tinydecode's example pairs Llama-3.2-3B with a Llama-3.2-1B
# draft at k = 5 (tinydecode README, "using it"); FlashSpec sweeps gamma over
# 1..16 with a Qwen2.5-1.5B target and a 0.5B drafter (FlashSpec page, results
# tables). Their vocabularies set V; 50257 is a size that is not a multiple
# of 4, which takes the library's scalar-load path.
#
# Stand-ins for model outputs: target logits are float32 N(0, sigma^2)
# (sigma = 3 gives a spread of about 27 over 128k entries, peaked like a
# language model's); the draft distribution q is the softmax of the target
# logits plus N(0, draft_noise^2) noise at the same temperature (a drafter
# that mostly agrees with its target); draft tokens are drawn from q with
# NumPy's choice; u and r are float32 uniforms in [0, 1).
# ---------------------------------------------------------------------------

SPEC_VOCABS = {"llama3": 128256, "qwen2.5": 151936, "ragged": 50257}


def spec_sampling_case(B: int, T: int, V: int, seed: int, *, tau: float = 1.0, sigma: float = 3.0,
                       draft_noise: float = 1.0, ctx_max: int = 8192) -> dict:
    """Seeded inputs of one sampling step: logits [B][T][V], q [B][T-1][V],
    drafts [B][T-1], u [B][T-1], r [B], ctx [B], tau (a float32 value)."""
    rng = np.random.default_rng(seed)
    G = T - 1
    logits = rng.standard_normal((B, T, V), dtype=np.float32) * np.float32(sigma)
    tau = float(np.float32(tau))
    q = np.zeros((B, G, V), dtype=np.float32)
    drafts = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        for i in range(G):
            z = (logits[b, i].astype(np.float64) + rng.standard_normal(V) * draft_noise) / tau
            e = np.exp(z - z.max())
            q64 = e / e.sum()
            q[b, i] = q64
            drafts[b, i] = rng.choice(V, p=q64)
    u = rng.random((B, G), dtype=np.float32)
    r = rng.random(B, dtype=np.float32)
    ctx = rng.integers(0, ctx_max, B).astype(np.int32)
    return {"logits": logits, "q": q, "drafts": drafts, "u": u, "r": r, "ctx": ctx, "tau": tau}


def spec_greedy_case(B: int, T: int, V: int, seed: int, *, sigma: float = 3.0, tie_frac: float = 0.25,
                     ctx_max: int = 8192) -> dict:
    """Seeded inputs of one greedy step with planted maxima.

    Position i of row b gets one entry raised 1 above the row's largest
    logit (in a `tie_frac` share of positions, two entries share that value:
    the top token is then the smaller index). The drafts equal the top tokens
    of the first m[b] positions (m uniform in 0..T-1) and differ from it at
    position m[b]. Returns the step's inputs plus `top` [B][T] and `m` [B]."""
    rng = np.random.default_rng(seed)
    G = T - 1
    logits = rng.standard_normal((B, T, V), dtype=np.float32) * np.float32(sigma)
    top = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        for i in range(T):
            hi = np.float32(logits[b, i].max() + 1)
            g = int(rng.integers(V))
            logits[b, i, g] = hi
            if V > 1 and rng.random() < tie_frac:
                g2 = int((g + 1 + rng.integers(V - 1)) % V)
                logits[b, i, g2] = hi
                g = min(g, g2)
            top[b, i] = g
    m = rng.integers(0, T, B).astype(np.int32)
    drafts = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        for i in range(G):
            drafts[b, i] = top[b, i] if i < m[b] else (top[b, i] + 1 + rng.integers(max(V - 1, 1))) % V
    ctx = rng.integers(0, ctx_max, B).astype(np.int32)
    return {"logits": logits, "drafts": drafts, "ctx": ctx, "tau": 0.0, "top": top, "m": m}
