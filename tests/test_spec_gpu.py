"""HIP speculative accept/reject + rollback vs the fp64 oracle, through the C ABI.

Greedy steps (tau = 0) are integer work on fp32 comparisons: the accept
counts, tokens and new lengths must equal the oracle's bit for bit, and the
planted top tokens of the inputs.

Sampling steps take their decisions from floating point: the kernel works in
fp32 (log2 space), the oracle in fp64. A decision whose fp64 margin is wider
than the kernel's rounding bound must come out the same; inside that bound
either outcome is correct, and the test then checks the result is one of them.
Bounds (derived from the kernel's arithmetic):
  * keep/reject: the kernel's log p(d) - log q(d) - log u differs from the
    exact one by a few ulps of |l_d - max| * log2(e)/tau, of log2 of the
    softmax sum (at most ~60 roundings of terms each within ~3 ulps), and of
    log2 q and log2 u: below 2e-5 (natural log) for these inputs. A decision
    is a near-tie when |ln u - (ln p(d) - ln q(d))| < DELTA_ACC = 2e-4.
  * the draw: each weight's absolute error is below 1e-5 * p_k plus its
    rounding, the running sums and the threshold r * total add at most ~60
    roundings of numbers <= 1: the kernel's running sums and threshold are
    within 3e-5 of the exact ones. A draw is a near-tie when the oracle's
    threshold lies within DELTA_S = 3e-4 of either end of the chosen token's
    interval; the kernel's token must then have an interval within DELTA_S
    of the threshold.
Near-ties must stay rare (a handful per thousand rows); every other row must
match exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads

pytestmark = pytest.mark.gpu

DELTA_ACC = 2e-4
DELTA_S = 3e-4
LLAMA3_V = workloads.SPEC_VOCABS["llama3"]
QWEN_V = workloads.SPEC_VOCABS["qwen2.5"]
RAGGED_V = workloads.SPEC_VOCABS["ragged"]


def _dev(a, dtype=None):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(case, S_max, ws=None, stream=None):
    logits = case["logits"]
    B, T, V = logits.shape
    G = T - 1
    greedy = case["tau"] == 0
    lens = _dev(case["ctx"].astype(np.int32))
    res = torch.full((B, 2), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = torch.empty(sda.spec_accept_workspace_bytes(B, T, V), dtype=torch.uint8, device="cuda")
    sda.spec_accept(_dev(logits), None if greedy or G == 0 else _dev(case["q"]),
                    _dev(case["drafts"]) if G > 0 else None, None if greedy or G == 0 else _dev(case["u"]),
                    None if greedy else _dev(case["r"]), case["tau"], lens, res, ws, S_max, stream=stream)
    torch.cuda.synchronize()
    r = res.cpu().numpy()
    return r[:, 0].copy(), r[:, 1].copy(), lens.cpu().numpy()


def _oracle(case, S_max):
    traces = []
    n, k, lens = oracle.accept_reject(case["logits"], case.get("q"), case["drafts"], case.get("u"),
                                      case.get("r"), case["tau"], case["ctx"], S_max, traces)
    return n, k, lens, traces


def _compare(case, S_max, got, max_tie_frac=0.02):
    """Exact match where the decisions are clear; a valid outcome at near-ties."""
    gn, gk, glen = got
    on, ok, olen, traces = _oracle(case, S_max)
    B, T, V = case["logits"].shape
    assert np.all((gn >= 0) & (gn <= T - 1)) and np.all((gk >= 0) & (gk < V))
    # the length is always the rollback of the kernel's own accept count
    assert np.array_equal(glen, [oracle.new_length(c, n, S_max) for c, n in zip(case["ctx"], gn)])
    if case["tau"] == 0:
        assert np.array_equal(gn, on) and np.array_equal(gk, ok)
        return 0
    ties = 0
    for b in range(B):
        if gn[b] == on[b] and gk[b] == ok[b]:
            continue
        tr = traces[b]
        margins = [abs(lu - lr) for lu, lr in zip(tr["log_u"], tr["log_ratio"])
                   if math.isfinite(lu) and math.isfinite(lr)]
        if margins and min(margins) < DELTA_ACC:
            ties += 1
            continue
        assert gn[b] == on[b], f"row {b}: accepted {gn[b]} vs {on[b]} with clear margins {margins}"
        w, c, t = tr["weights"], tr["cum"], tr["t"]
        k, kk = int(ok[b]), int(gk[b])
        assert min(t - (c[k] - w[k]), c[k] - t) < DELTA_S, f"row {b}: token {kk} vs {k}, clear draw"
        assert c[kk] - w[kk] - DELTA_S <= t <= c[kk] + DELTA_S and w[kk] > -DELTA_S, f"row {b}: token {kk} invalid"
        ties += 1
    assert ties <= max(1, int(max_tie_frac * B)), f"{ties} near-ties in {B} rows"
    return ties


# ------------------------------------------------------------------ greedy

@pytest.mark.parametrize("B,T,V", [(16, 6, LLAMA3_V), (8, 6, RAGGED_V), (5, 17, QWEN_V), (3, 32, 3000),
                                   (64, 6, 7), (4, 1, LLAMA3_V)])
def test_greedy_matches_oracle_and_planted_tokens(B, T, V):
    case = workloads.spec_greedy_case(B, T, V, seed=900 + T + V % 97)
    S_max = 16384
    got = _run(case, S_max)
    _compare(case, S_max, got)
    n, k, _ = got
    assert np.array_equal(n, case["m"])
    assert np.array_equal(k, case["top"][np.arange(B), case["m"]])


# ---------------------------------------------------------------- sampling

@pytest.mark.parametrize("B,T,V,tau", [
    (16, 6, LLAMA3_V, 1.0),       # Llama-3.2-3B verify step, k = 5
    (8, 6, LLAMA3_V, 0.7),
    (6, 9, QWEN_V, 1.0),          # Qwen2.5 vocabulary, gamma = 8
    (8, 6, RAGGED_V, 1.0),        # V % 4 != 0: scalar loads
    (4, 17, 20000, 0.5),          # gamma = 16
    (2, 32, 5000, 1.3),           # the largest T
    (12, 1, LLAMA3_V, 1.0),       # no drafts: a plain sample from p_0
    (3, 6, 1, 1.0),               # one-token vocabulary
    (200, 3, 97, 1.0),            # many small rows
])
def test_sampling_matches_oracle(B, T, V, tau):
    case = workloads.spec_sampling_case(B, T, V, seed=1000 + B + T + V % 101, tau=tau)
    S_max = 16384
    _compare(case, S_max, _run(case, S_max))


def test_sampling_full_batch_llama3():
    """64 rows of the Llama-3 vocabulary at k = 5, the launch shape the bench
    times (every row checked)."""
    case = workloads.spec_sampling_case(64, 6, LLAMA3_V, seed=1111)
    _compare(case, 16384, _run(case, 16384))


# ------------------------------------------------------------- edge cases

def test_zero_u_or_zero_q_keeps_and_bad_ids_reject():
    case = workloads.spec_sampling_case(6, 6, 3000, seed=1200)
    case["u"][0] = 0.0                                  # u = 0 keeps everything
    case["q"][1, 2, case["drafts"][1, 2]] = 0.0         # q(d) = 0 keeps draft 2 of row 1
    case["u"][1, :2] = 0.0
    case["drafts"][2, 1] = -1                           # out of range: rejected at 1
    case["u"][2, 0] = 0.0
    case["drafts"][3, 0] = 3000
    case["drafts"][4, 3] = 2 ** 31 - 1
    case["u"][4, :3] = 0.0
    got = _run(case, 16384)
    _compare(case, 16384, got)
    n = got[0]
    assert n[0] == 5 and n[1] >= 3 and n[2] == 1 and n[3] == 0 and n[4] == 3


def test_masked_vocabulary_entries():
    """-inf logits (padded vocabulary): never drawn, never kept."""
    for tau in (0.0, 1.0):
        case = (workloads.spec_greedy_case(8, 6, 4099, seed=1300) if tau == 0
                else workloads.spec_sampling_case(8, 6, 4099, seed=1301))
        case["logits"][:, :, 4000:] = -np.inf
        if tau:
            case["drafts"][0, 0] = 4050                 # a masked draft: p(d) = 0, rejected
        got = _run(case, 16384)
        _compare(case, 16384, got)
        assert np.all(got[1] < 4000)


def test_length_rollback_clamps():
    case = workloads.spec_greedy_case(6, 6, 1000, seed=1400)
    S_max = 100
    case["ctx"][:] = [0, -7, 99, 100, 250, 94]
    got = _run(case, S_max)
    _compare(case, S_max, got)
    assert got[2][1] == case["m"][1] + 1 and got[2][2] == 100 and got[2][3] == 100


# ----------------------------------------------- reuse and graph capture

def test_workspace_reused_by_calls_of_different_shapes():
    big = workloads.spec_sampling_case(32, 6, 9000, seed=1500)
    small = workloads.spec_sampling_case(5, 4, 70000, seed=1501)
    ws = torch.empty(max(sda.spec_accept_workspace_bytes(32, 6, 9000), sda.spec_accept_workspace_bytes(5, 4, 70000)),
                     dtype=torch.uint8, device="cuda")
    for case in (big, small, big, small):
        _compare(case, 16384, _run(case, 16384, ws=ws))


def test_graph_replays_with_new_inputs():
    B, T, V, S_max = 8, 6, 30000, 16384
    first = workloads.spec_sampling_case(B, T, V, seed=1600)
    bufs = {k: _dev(first[k]) for k in ("logits", "q", "drafts", "u", "r", "ctx")}
    res = torch.empty((B, 2), dtype=torch.int32, device="cuda")
    ws = torch.empty(sda.spec_accept_workspace_bytes(B, T, V), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sda.spec_accept(bufs["logits"], bufs["q"], bufs["drafts"], bufs["u"], bufs["r"], first["tau"],
                        bufs["ctx"], res, ws, S_max, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            sda.spec_accept(bufs["logits"], bufs["q"], bufs["drafts"], bufs["u"], bufs["r"], first["tau"],
                            bufs["ctx"], res, ws, S_max, stream=s)
    for rep in range(3):
        case = workloads.spec_sampling_case(B, T, V, seed=1610 + rep)
        with torch.cuda.stream(s):
            for k in ("logits", "q", "drafts", "u", "r", "ctx"):
                bufs[k].copy_(_dev(case[k]))
            g.replay()
        s.synchronize()
        r = res.cpu().numpy()
        _compare(case, S_max, (r[:, 0].copy(), r[:, 1].copy(), bufs["ctx"].cpu().numpy()))


# --------------------------------- the pages' distribution check, on the GPU

P_CHI = np.array([0.30, 0.25, 0.20, 0.12, 0.08, 0.05])
Q_CHI = np.array([0.10, 0.15, 0.20, 0.25, 0.20, 0.10])


def _chi_case(N, gamma, rng):
    logits = np.broadcast_to(np.log(P_CHI).astype(np.float32), (N, gamma + 1, 6)).copy()
    q = np.broadcast_to(Q_CHI.astype(np.float32), (N, gamma, 6)).copy()
    drafts = np.minimum(np.searchsorted(np.cumsum(Q_CHI), rng.random((N, gamma)), side="right"), 5).astype(np.int32)
    return {"logits": logits, "q": q, "drafts": drafts, "u": rng.random((N, gamma), dtype=np.float32),
            "r": rng.random(N, dtype=np.float32), "ctx": np.zeros(N, np.int32), "tau": 1.0}


@pytest.mark.parametrize("gamma", [1, 4])
def test_emitted_tokens_follow_target_chi_squared(gamma):
    """The FlashSpec CI check (N = 30000, vocabulary 6, 1% point 15.086 at 5
    degrees of freedom) on tokens the HIP kernels emit, first token and, for
    gamma 4, the second (rows that kept no draft take a second step)."""
    N = 30000
    rng = np.random.default_rng(1700 + gamma)
    case = _chi_case(N, gamma, rng)
    n, k, _ = _run(case, 1 << 20)
    first = np.where(n >= 1, case["drafts"][:, 0], k)
    chi = lambda toks: float((((np.bincount(toks, minlength=6) - N * P_CHI) ** 2) / (N * P_CHI)).sum())
    assert chi(first) < 15.086
    sub = np.arange(0, N, 10)                           # 3000 rows against the oracle
    _compare({key: (v[sub] if isinstance(v, np.ndarray) else v) for key, v in case.items()}, 1 << 20,
             (n[sub], k[sub], np.array([oracle.new_length(0, x, 1 << 20) for x in n[sub]])))
    if gamma == 4:
        again = np.flatnonzero(n == 0)
        step2 = _chi_case(len(again), gamma, rng)
        n2, k2, _ = _run(step2, 1 << 20)
        second = np.where(n >= 2, case["drafts"][:, 1], k)
        second[again] = np.where(n2 >= 1, step2["drafts"][:, 0], k2)
        assert chi(second) < 15.086


@pytest.mark.parametrize("V", [(1 << 21) + 4, (1 << 21) + 3])
def test_vocabulary_past_the_chunk_cap(V):
    """More than 2048 chunks of 1024 entries: the chunks widen to stay within
    the LDS stage of the decision (and V % 4 != 0 takes the scalar loads)."""
    case = workloads.spec_sampling_case(2, 3, V, seed=1800 + V % 7)
    _compare(case, 16384, _run(case, 16384))
    g = workloads.spec_greedy_case(2, 3, V, seed=1810 + V % 7)
    got = _run(g, 16384)
    _compare(g, 16384, got)
    assert np.array_equal(got[0], g["m"])
