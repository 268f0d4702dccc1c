"""fp64 oracle for the accept/reject step of speculative decoding and the
on-device rollback of the cache lengths.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain NumPy, sharing
nothing with the HIP library.

What the pages fix:
  * each draft survives with probability min(1, p_t / p_d); at the first
    one that does not, the step's extra token is drawn from the positive part
    of p_t - p_d, and when all survive, from the target's last (bonus) row;
    with temperature 0 the survivors are the leading drafts that match the
    target's argmax (tinydecode README, "speculative decoding");
  * the test is u_i < min(1, p(x_i) / q(x_i)), evaluated in log space, and a
    rejected position draws its token from max(0, p - q) normalised to sum 1
    (Leviathan et al. 2023, Algorithm 1, as the FlashSpec page restates it in
    its correctness paragraph); greedy mode keeps the longest prefix that
    matches the target's argmax (FlashSpec page, "What is FlashSpec?");
  * one read of the accept count and the next token per step, and rollback of
    a static cache by moving the length only: entries past it are never read
    (tinydecode README, "speculative decoding"; FlashSpec page, compiled path).

Readings taken where the pages are silent (restated where used):
  S1. Inputs of row b: target logits [T][V] (fp32) for the T = gamma + 1
      positions of the verify pass -- position i scores the token that follows
      draft i-1, position 0 the token after the pending one, and position gamma
      is the bonus row; the gamma draft tokens; the draft probabilities q
      [gamma][V] (fp32) those tokens were drawn from; uniforms u [gamma] and
      one uniform r for the extra token (random draws are inputs); a
      temperature tau shared by the batch; the row's cache length ctx before
      the verify pass.
  S2. p_i = softmax(logits_i / tau), worked in fp64 from the fp32 logits.
  S3. Draft i is kept iff ln u_i < ln p_i(d_i) - ln q_i(d_i), with ln 0 = -inf
      (so u_i = 0 or q_i(d_i) = 0 keeps it). A draft id outside [0, V) is
      rejected.
  S4. The extra token is drawn by inverse CDF in index order: with weights w
      (the residual, or p_gamma for the bonus) and t = r * sum(w), it is the
      first index k with w_k > 0 whose running sum exceeds t; if rounding puts
      t at or past the total, the last index with w_k > 0. A residual with no
      positive weight (only reachable through rounding) is replaced by p of
      that position.
  S5. tau = 0: draft i is kept while it equals argmax_k logits_i[k] (smallest
      index on ties); the extra token is the argmax of the first position not
      kept (the bonus row when all were).
  S6. The new length is min(clamp(ctx, 0, S_max) + n + 1, S_max): the pending
      token and the n kept drafts stay in the cache; the rejected drafts'
      entries lie past the new length; the extra token becomes the next pending
      token and is not in the cache yet.
"""
from __future__ import annotations

import math

import numpy as np


def argmax_first(row) -> int:
    """Index of the largest value, the smallest such index on ties (S5)."""
    row = np.asarray(row)
    return int(np.flatnonzero(row == row.max())[0])


def log_target_probs(logits_row, tau: float) -> np.ndarray:
    """ln p with p = softmax(logits / tau), in float64 (S2)."""
    z = np.asarray(logits_row, dtype=np.float64) / float(tau)
    z = z - z.max()
    return z - math.log(np.exp(z).sum())


def target_probs(logits_row, tau: float) -> np.ndarray:
    """p = softmax(logits / tau) in float64 (S2)."""
    return np.exp(log_target_probs(logits_row, tau))


def _ln(x: float) -> float:
    return -math.inf if x <= 0.0 else math.log(x)


def sample_index(w, r: float, trace=None) -> int:
    """Inverse-CDF draw in index order (S4)."""
    w = np.asarray(w, dtype=np.float64)
    total = w.sum()
    t = float(r) * total
    c = np.cumsum(w)
    hit = np.flatnonzero((c > t) & (w > 0))
    k = int(hit[0]) if hit.size else int(np.flatnonzero(w > 0)[-1])
    if trace is not None:
        trace.update(weights=w, cum=c, t=t)
    return k


def accept_reject_row(logits, q, drafts, u, r: float, tau: float, trace=None):
    """One row of the step (S1-S5): returns (n kept, next token).

    If `trace` is a dict it receives, for every position examined, the log
    ratio ln p(d) - ln q(d) and ln u (sampling) or the argmax (greedy), and
    the weights, running sums and threshold of the final draw.
    """
    logits = np.asarray(logits)
    T, V = logits.shape
    gamma = T - 1
    if tau == 0:
        n = 0
        while n < gamma and int(drafts[n]) == argmax_first(logits[n]):
            n += 1
        return n, argmax_first(logits[n])
    log_ratio, log_u = [], []
    n = gamma
    for i in range(gamma):
        d = int(drafts[i])
        if not 0 <= d < V:
            log_ratio.append(-math.inf)
            log_u.append(_ln(float(u[i])))
            n = i
            break
        lp = log_target_probs(logits[i], tau)
        lr = float(lp[d]) - _ln(float(q[i][d]))
        lu = _ln(float(u[i]))
        log_ratio.append(lr)
        log_u.append(lu)
        if not lu < lr:
            n = i
            break
    if trace is not None:
        trace.update(log_ratio=log_ratio, log_u=log_u)
    p = target_probs(logits[n], tau)
    if n < gamma:
        w = np.maximum(0.0, p - np.asarray(q[n], dtype=np.float64))
        if not np.any(w > 0):
            w = p
    else:
        w = p
    return n, sample_index(w, r, trace)


def new_length(ctx: int, n: int, S_max: int) -> int:
    """Rollback of the cache length (S6)."""
    return min(min(max(int(ctx), 0), S_max) + n + 1, S_max)


def accept_reject(logits, q, drafts, u, r, tau: float, ctx_lens, S_max: int, traces=None):
    """Every row of the step (S1-S6).

    logits float32 [B][T][V]; q float32 [B][T-1][V]; drafts int [B][T-1];
    u float32 [B][T-1]; r float32 [B]; ctx_lens int [B]; q, u and r may be
    None when tau == 0.
    Returns (n_kept int32 [B], next_token int32 [B], new_lens int32 [B]).
    `traces`, if a list, receives one trace dict per row.
    """
    logits = np.asarray(logits, dtype=np.float32)
    B = logits.shape[0]
    n_acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        tr = {} if traces is not None else None
        n, k = accept_reject_row(logits[b], None if q is None else q[b], drafts[b],
                                 None if u is None else u[b], 0.0 if r is None else float(r[b]), float(tau), tr)
        n_acc[b], nxt[b] = n, k
        lens[b] = new_length(ctx_lens[b], n, S_max)
        if traces is not None:
            traces.append(tr)
    return n_acc, nxt, lens
