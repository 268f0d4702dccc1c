"""Pins for the speculative accept/reject + rollback oracle (CPU only).

The pages print no worked example for this step, so the oracle is pinned by:
  * hand-worked cases of Algorithm 1 (Leviathan et al. 2023), with
    distributions whose ratios and residuals are exact small fractions;
  * the check the FlashSpec page describes for its CI: emitted tokens follow
    the target distribution p when the draft distribution q differs from it,
    a Pearson chi-squared test over a 6-token vocabulary, N = 30000, gamma 1
    and 4 (first emitted token, and the second one for gamma 4), against the
    1% point of chi-squared with 5 degrees of freedom, 15.086
    (Theorem 1 of the same paper);
  * tinydecode's greedy check: at temperature 0 the accepted drafts plus the
    extra token are exactly what plain greedy decoding of the target emits;
  * closed forms: the accepted fraction of a grid of uniforms is
    min(1, p(d)/q(d)); the residual draw over a grid of uniforms lands on k
    with frequency max(0, p_k - q_k) / sum; draft == target accepts all;
    a huge temperature makes p uniform;
  * mutation tests: plausible mistakes planted in a copy of the oracle must
    each fail one of these pins.
"""
from __future__ import annotations

import importlib
import math
import types

import numpy as np
import pytest
from scipy.special import softmax

ospec = importlib.import_module("oracle.speculative")

CHI2_CRIT_5DOF_1PCT = 15.086


def _ln32(values):
    return np.log(np.asarray(values, dtype=np.float64)).astype(np.float32)


def _f32(values):
    return np.asarray(values, dtype=np.float32)


# ------------------------------------------------------------ hand-worked

def _hand_case():
    # position 0: p = [1/2, 1/4, 1/8, 1/8]; q = [1/4, 1/2, 1/8, 1/8]; draft 1
    #   -> ratio p/q = 1/2, residual max(0, p - q) = [1/4, 0, 0, 0]
    # position 1: p uniform; q = [0.1, 0.2, 0.3, 0.4]; draft 3
    #   -> ratio 0.25 / 0.4 = 0.625, residual = [0.15, 0.05, 0, 0]
    # position 2 (bonus): p = [0.1, 0.2, 0.3, 0.4]
    logits = np.stack([_ln32([4, 2, 1, 1]), _ln32([1, 1, 1, 1]), _ln32([1, 2, 3, 4])])
    q = _f32([[0.25, 0.5, 0.125, 0.125], [0.1, 0.2, 0.3, 0.4]])
    return logits, q, [1, 3]


@pytest.mark.parametrize("u,r,want", [
    ((0.6, 0.0), 0.9, (0, 0)),     # reject draft 0 (0.6 >= 1/2): residual has one token
    ((0.4, 0.7), 0.5, (1, 0)),     # keep 0, reject 1; t = 0.1 of residual mass 0.2 -> token 0
    ((0.4, 0.7), 0.8, (1, 1)),     # t = 0.16 > 0.15 -> token 1
    ((0.4, 0.6), 0.35, (2, 2)),    # keep both; bonus p = [.1,.2,.3,.4], t = 0.35 -> token 2
    ((0.4, 0.6), 0.05, (2, 0)),
    ((0.0, 0.0), 0.95, (2, 3)),    # u = 0 always keeps
])
def test_hand_worked_sampling(u, r, want):
    logits, q, drafts = _hand_case()
    got = ospec.accept_reject_row(logits, q, drafts, _f32(u), r, 1.0)
    assert got == want


def test_hand_worked_batch_and_rollback():
    logits, q, drafts = _hand_case()
    L = np.stack([logits] * 3)
    Q = np.stack([q] * 3)
    D = np.array([drafts] * 3)
    U = _f32([[0.6, 0.0], [0.4, 0.7], [0.4, 0.6]])
    n, nxt, lens = ospec.accept_reject(L, Q, D, U, _f32([0.9, 0.8, 0.35]), 1.0,
                                       np.array([10, 20, 98]), S_max=100)
    assert n.tolist() == [0, 1, 2]
    assert nxt.tolist() == [0, 1, 2]
    assert lens.tolist() == [11, 22, 100]     # ctx + n + 1, capped at S_max


def test_new_length_rules():
    assert ospec.new_length(7, 0, 64) == 8
    assert ospec.new_length(7, 5, 64) == 13
    assert ospec.new_length(62, 5, 64) == 64
    assert ospec.new_length(-3, 2, 64) == 3
    assert ospec.new_length(500, 0, 64) == 64


def test_out_of_range_draft_is_rejected():
    logits, q, _ = _hand_case()
    # draft 0 is out of range: rejected at 0 whatever u says; residual of position 0
    assert ospec.accept_reject_row(logits, q, [4, 3], _f32([0.0, 0.0]), 0.9, 1.0) == (0, 0)
    assert ospec.accept_reject_row(logits, q, [1, -1], _f32([0.0, 0.0]), 0.8, 1.0) == (1, 1)
    assert ospec.accept_reject_row(logits, q, [-1, 3], _f32([0.0, 0.0]), 0.0, 0.0)[0] == 0


# --------------------------------------------------------- sample_index

def test_sample_index_hand_cases():
    w = [0.0, 0.5, 0.0, 0.5]
    assert ospec.sample_index(w, 0.0) == 1      # first index with positive weight
    assert ospec.sample_index(w, 0.25) == 1
    assert ospec.sample_index(w, 0.5) == 3      # running sum must exceed t
    assert ospec.sample_index(w, 0.999) == 3
    assert ospec.sample_index(w, 1.0) == 3      # t at the total: last positive index
    assert ospec.sample_index([0.0, 2.0, 6.0, 0.0], 0.25) == 2   # unnormalised weights
    assert ospec.sample_index([0.0, 2.0, 6.0, 0.0], 0.2499) == 1


def test_sample_index_frequencies_on_a_grid():
    rng = np.random.default_rng(5)
    w = rng.random(9) * (rng.random(9) > 0.3)
    M = 4000
    counts = np.bincount([ospec.sample_index(w, (j + 0.5) / M) for j in range(M)], minlength=9)
    assert np.all(counts[w == 0] == 0)
    assert np.max(np.abs(counts / M - w / w.sum())) <= 1.0 / M + 1e-12


# --------------------------------------------------- closed forms

def _probs(logits, tau=1.0):
    return softmax(np.asarray(logits, dtype=np.float64) / tau)


def test_acceptance_fraction_is_min_one_ratio():
    rng = np.random.default_rng(6)
    V, M = 7, 2000
    logits = rng.normal(size=(2, V)).astype(np.float32)
    q = _f32(_probs(rng.normal(size=V) * 1.5))[None, :]
    p = _probs(logits[0])
    for d in range(V):
        kept = sum(ospec.accept_reject_row(logits, q, [d], _f32([(j + 0.5) / M]), 0.5, 1.0)[0]
                   for j in range(M))
        assert abs(kept / M - min(1.0, p[d] / float(q[0, d]))) <= 1.0 / M + 1e-6


def test_residual_frequencies():
    rng = np.random.default_rng(7)
    V, M = 6, 3000
    logits = rng.normal(size=(2, V)).astype(np.float32)
    q = _f32(_probs(rng.normal(size=V)))[None, :]
    p = _probs(logits[0])
    d = int(np.argmax(q[0].astype(np.float64) - p))   # q(d) > p(d): rejection possible
    resid = np.maximum(0.0, p - q[0].astype(np.float64))
    counts = np.zeros(V)
    for j in range(M):
        n, k = ospec.accept_reject_row(logits, q, [d], _f32([0.9999999]), (j + 0.5) / M, 1.0)
        assert n == 0
        counts[k] += 1
    assert np.max(np.abs(counts / M - resid / resid.sum())) <= 1.0 / M + 1e-6


def test_draft_equal_to_target_keeps_everything():
    rng = np.random.default_rng(8)
    V, gamma = 50, 5
    logits = (rng.normal(size=(gamma + 1, V)) * 2).astype(np.float32)
    q = _f32([_probs(l, 0.7) for l in logits[:gamma]])
    for trial in range(20):
        drafts = [rng.choice(V, p=_probs(l, 0.7)) for l in logits[:gamma]]
        u = _f32(rng.random(gamma) * 0.999)
        n, k = ospec.accept_reject_row(logits, q, drafts, u, float(rng.random()), 0.7)
        assert n == gamma and 0 <= k < V


def test_huge_temperature_makes_target_uniform():
    rng = np.random.default_rng(9)
    V = 8
    logits = rng.normal(size=(2, V)).astype(np.float32)
    q = _f32(_probs(rng.normal(size=V)))[None, :]
    for d in range(V):
        for u in (0.1, 0.4, 0.7):
            n, _ = ospec.accept_reject_row(logits, q, [d], _f32([u]), 0.3, 1e9)
            assert n == int(u < (1.0 / V) / float(q[0, d]))


def test_temperature_divides_the_logits():
    rng = np.random.default_rng(10)
    V, gamma = 16, 3
    logits = rng.normal(size=(gamma + 1, V)).astype(np.float32)
    q = _f32([_probs(rng.normal(size=V)) for _ in range(gamma)])
    for t in range(30):
        drafts = rng.integers(0, V, gamma)
        u, r = _f32(rng.random(gamma)), float(rng.random())
        a = ospec.accept_reject_row(logits, q, drafts, u, r, 1.0)
        b = ospec.accept_reject_row(logits * np.float32(4), q, drafts, u, r, 4.0)
        assert a == b


# --------------------------------------------------- greedy vs plain greedy

def _greedy_sequence(table, start, steps):
    seq, tok = [], start
    for _ in range(steps):
        row = table[tok]
        tok = int(np.flatnonzero(row == row.max())[0])
        seq.append(tok)
    return seq


def test_greedy_equals_plain_greedy_decoding():
    """Toy target whose next-token logits depend on the previous token."""
    rng = np.random.default_rng(11)
    V, gamma = 12, 4
    table = rng.normal(size=(V, V)).astype(np.float32)
    table[3, 5] = table[3, 2] = table[3].max() + 1      # a tie: the smaller index wins
    for trial in range(200):
        pending = int(rng.integers(V))
        plain = _greedy_sequence(table, pending, gamma + 1)
        m = int(rng.integers(0, gamma + 1))             # drafts agree for m tokens
        drafts = list(plain[:m]) + [int(rng.integers(V)) for _ in range(gamma - m)]
        logits = np.stack([table[t] for t in [pending] + drafts])
        n, k = ospec.accept_reject_row(logits, None, drafts, None, 0.0, 0.0)
        emitted = drafts[:n] + [k]
        assert emitted == plain[:n + 1]
        assert n == gamma or drafts[n] != plain[n]       # the longest matching prefix
    assert _greedy_sequence(table, 3, 1) == [2]


# --------------------------------------------------- chi-squared (Theorem 1)

P_CHI = np.array([0.30, 0.25, 0.20, 0.12, 0.08, 0.05])
Q_CHI = np.array([0.10, 0.15, 0.20, 0.25, 0.20, 0.10])


def _chi2(counts, p):
    N = counts.sum()
    return float(((counts - N * p) ** 2 / (N * p)).sum())


def _emitted_pairs(mod, gamma, N, seed):
    """First two emitted tokens of N independent generations whose every
    position has target p and draft q."""
    rng = np.random.default_rng(seed)
    V = len(P_CHI)
    logits = np.stack([_ln32(P_CHI)] * (gamma + 1))
    q = np.stack([_f32(Q_CHI)] * gamma)
    cq = np.cumsum(Q_CHI)
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    for _ in range(N):
        out = []
        while len(out) < 2:
            drafts = np.minimum(np.searchsorted(cq, rng.random(gamma), side="right"), V - 1)
            n, k = mod.accept_reject_row(logits, q, drafts, _f32(rng.random(gamma)),
                                         float(rng.random()), 1.0)
            out += [int(t) for t in drafts[:n]] + [k]
        first[out[0]] += 1
        second[out[1]] += 1
    return first, second


@pytest.mark.parametrize("gamma", [1, 4])
def test_emitted_tokens_follow_target_chi_squared(gamma):
    first, second = _emitted_pairs(ospec, gamma, 30000, 1000 + gamma)
    assert _chi2(first, P_CHI) < CHI2_CRIT_5DOF_1PCT
    if gamma == 4:
        assert _chi2(second, P_CHI) < CHI2_CRIT_5DOF_1PCT
    # and the draft distribution alone would fail it badly
    assert _chi2(np.round(Q_CHI * 30000), P_CHI) > 100 * CHI2_CRIT_5DOF_1PCT


# ------------------------------------------------------- mutation tests

def _battery(mod) -> list[str]:
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:
            failed.append(name + "-raised")

    logits, q, drafts = _hand_case()
    hand = [((0.6, 0.0), 0.9, (0, 0)), ((0.4, 0.7), 0.5, (1, 0)), ((0.4, 0.7), 0.8, (1, 1)),
            ((0.4, 0.6), 0.35, (2, 2)), ((0.9, 0.9), 0.5, (0, 0))]
    check("hand", lambda: all(mod.accept_reject_row(logits, q, drafts, _f32(u), r, 1.0) == w
                              for u, r, w in hand))
    check("sample", lambda: [mod.sample_index([0.0, 0.5, 0.0, 0.5], r) for r in (0.0, 0.5, 1.0)] == [1, 3, 3])
    check("length", lambda: mod.new_length(7, 2, 64) == 10 and mod.new_length(62, 5, 64) == 64)

    def tau():
        rng = np.random.default_rng(12)
        L = rng.normal(size=(3, 10)).astype(np.float32)
        Q = _f32([_probs(rng.normal(size=10)) for _ in range(2)])
        for _ in range(10):
            d, u, r = rng.integers(0, 10, 2), _f32(rng.random(2)), float(rng.random())
            if mod.accept_reject_row(L, Q, d, u, r, 1.0) != mod.accept_reject_row(L * np.float32(3), Q, d, u, r, 3.0):
                return False
        return True
    check("tau", tau)

    def greedy():
        rng = np.random.default_rng(13)
        V = 10
        table = rng.normal(size=(V, V)).astype(np.float32)
        table[4, 7] = table[4, 1] = table[4].max() + 1
        for pending in range(V):
            plain = _greedy_sequence(table, pending, 4)
            for m in range(4):
                drafts = plain[:m] + [(plain[m] + 1) % V] * (3 - m) if m < 3 else plain[:3]
                L = np.stack([table[t] for t in [pending] + drafts])
                n, k = mod.accept_reject_row(L, None, drafts, None, 0.0, 0.0)
                if drafts[:n] + [k] != plain[:n + 1]:
                    return False
        return True
    check("greedy", greedy)

    def chi():
        first, second = _emitted_pairs(mod, 4, 3000, 77)
        return _chi2(first, P_CHI) < CHI2_CRIT_5DOF_1PCT and _chi2(second, P_CHI) < CHI2_CRIT_5DOF_1PCT
    check("chi2", chi)
    return failed


MUTANTS = {
    "accept-when-u-exceeds": ("if not lu < lr:", "if lu < lr:"),
    "ratio-sign": ("lr = float(lp[d]) - _ln(", "lr = float(lp[d]) + _ln("),
    "residual-q-minus-p": ("w = np.maximum(0.0, p - np.asarray(q[n], dtype=np.float64))",
                           "w = np.maximum(0.0, np.asarray(q[n], dtype=np.float64) - p)"),
    "residual-is-p": ("w = np.maximum(0.0, p - np.asarray(q[n], dtype=np.float64))", "w = p"),
    "bonus-from-last-draft-row": ("p = target_probs(logits[n], tau)",
                                  "p = target_probs(logits[min(n, gamma - 1)], tau)"),
    "tau-multiplies": ("z = np.asarray(logits_row, dtype=np.float64) / float(tau)",
                       "z = np.asarray(logits_row, dtype=np.float64) * float(tau)"),
    "greedy-extra-from-next-row": ("return n, argmax_first(logits[n])",
                                   "return n, argmax_first(logits[min(n + 1, gamma)])"),
    "argmax-last-on-ties": ("return int(np.flatnonzero(row == row.max())[0])",
                            "return int(np.flatnonzero(row == row.max())[-1])"),
    "sample-at-or-above": ("hit = np.flatnonzero((c > t) & (w > 0))",
                           "hit = np.flatnonzero((c >= t) & (w > 0))"),
    "length-drops-pending": ("0), S_max) + n + 1, S_max)", "0), S_max) + n, S_max)"),
    "keeps-going-after-reject": ("            n = i\n            break\n    if trace",
                                 "            n = i\n    if trace"),
    "log-u-not-taken": ("lu = _ln(float(u[i]))", "lu = float(u[i])"),
}


def _load_mutant(old, new):
    src = open(ospec.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("spec_mutant")
    exec(compile(src.replace(old, new, 1), "spec_mutant", "exec"), mod.__dict__)
    return mod


def test_battery_passes_on_oracle():
    assert _battery(ospec) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    with np.errstate(all="ignore"):
        failed = _battery(_load_mutant(old, new))
    assert failed, f"mutant {name} passed every pin"
