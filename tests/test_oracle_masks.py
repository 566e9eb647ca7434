"""Pins for the oracle's rank / threshold / kept-set / decode-membership logic.

Each test checks the oracle against something other than itself: values worked
by hand from the definitions (tests/golden/), an independent characterisation
of the top-k set (dominance), exhaustive enumeration of tiny cases, closed forms
for monotone priorities, and the invariants the method fixes (row size
min(q+1, B), a non-increasing cutoff, evicted tokens never returning).
"""
import itertools
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_masks.txt")


def _parse_golden():
    cases, cur = [], None
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line == "case":
            cur = {"held": []}
            continue
        if line == "end":
            cases.append(cur)
            continue
        key, *vals = line.split()
        if key in ("S", "s", "w", "k"):
            cur[key] = int(vals[0])
        elif key == "prio":
            cur[key] = np.array([float(v) for v in vals], dtype=np.float32)
        elif key in ("rank", "tau"):
            cur[key] = np.array([orc.INT32_MAX if v == "MAX" else int(v) for v in vals])
        elif key == "held":
            cur["held"].append([int(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _parse_golden(), ids=lambda c: f"S{c['S']}s{c['s']}w{c['w']}k{c['k']}")
def test_hand_worked_examples(case):
    S, s, w, k, prio = case["S"], case["s"], case["w"], case["k"], case["prio"]
    rank = orc.priority_rank(prio)
    assert rank.tolist() == case["rank"].tolist()
    r2, tau = orc.thresholds_by_sorting(prio[None], s, w, k)
    assert tau[0].tolist() == case["tau"].tolist()
    tau_sel = orc.thresholds_by_selection(rank[None], s, w, k)
    assert tau_sel[0].tolist() == case["tau"].tolist()
    m = orc.mask_rows(rank, case["tau"], np.arange(S), s, w)
    for q in range(S):
        assert np.flatnonzero(m[q]).tolist() == case["held"][q], q
        assert orc.kept_row_by_sorting(prio, q, s, w, k).tolist() == case["held"][q]
    table = np.asarray(prio, dtype=np.float64)
    held, _ = orc.decode_simulate(table, s, w, k, S)
    for q in range(S):
        assert held[q].tolist() == case["held"][q], q


def _beats(p, a, b):
    """a is ahead of b in the order (priority desc, NaN lowest, index asc)."""
    pa = -np.inf if np.isnan(p[a]) else p[a]
    pb = -np.inf if np.isnan(p[b]) else p[b]
    return pa > pb or (pa == pb and a < b)


def _check_row(prio, q, s, w, k):
    """Independent characterisation: the long-range kept set L of row q is the
    subset of E(q) with |L| = min(k, |E|) such that every member beats every
    non-member."""
    E = list(range(s, max(s, q - w + 1)))
    L = orc.kept_long_by_sorting(prio, q, s, w, k)
    assert len(L) == min(k, len(E))
    assert set(L) <= set(E)
    for a in L:
        for b in set(E) - set(L):
            assert _beats(prio, a, b)
    return L


@pytest.mark.parametrize("S,s,w,k", [(6, 0, 1, 2), (6, 1, 2, 1), (6, 2, 1, 3), (7, 1, 1, 2),
                                     (5, 0, 2, 0), (5, 1, 1, 9)])
def test_exhaustive_permutations(S, s, w, k):
    B = s + w + k
    for perm in itertools.permutations(range(S)):
        prio = np.array(perm, dtype=np.float32) * 0.5 - 1.0
        rank = orc.priority_rank(prio)
        _, tau = orc.thresholds_by_sorting(prio[None], s, w, k)
        tau = tau[0]
        m = orc.mask_rows(rank, tau, np.arange(S), s, w)
        held, st = orc.decode_simulate(prio.astype(np.float64), s, w, k, S)
        for q in range(S):
            L = _check_row(prio, q, s, w, k)
            row = np.flatnonzero(m[q])
            assert len(row) == min(q + 1, B)
            expect = sorted(set(range(min(s, q + 1))) | set(range(max(0, q - w + 1), q + 1)) | set(L))
            assert row.tolist() == expect
            assert held[q].tolist() == expect
        assert not (st.evicted & set(held[S - 1].tolist()))


def test_tie_heavy_fuzz():
    rng = np.random.default_rng(11)
    for trial in range(60):
        S = int(rng.integers(1, 40))
        s, w, k = int(rng.integers(0, 5)), int(rng.integers(1, 6)), int(rng.integers(0, 8))
        prio = np.round(rng.standard_normal(S) * 1.5).astype(np.float32)  # many ties
        if trial % 5 == 0:
            prio[rng.integers(0, S, size=max(1, S // 6))] = np.nan
        if trial % 7 == 0:
            prio[prio == 0] = -0.0
        rank = orc.priority_rank(prio)
        assert sorted(rank.tolist()) == list(range(S))
        _, tau = orc.thresholds_by_sorting(prio[None], s, w, k)
        tau_sel = orc.thresholds_by_selection(rank[None], s, w, k)
        assert tau.tolist() == tau_sel.tolist()
        m = orc.mask_rows(rank, tau[0], np.arange(S), s, w)
        held, _ = orc.decode_simulate(prio.astype(np.float64), s, w, k, S)
        for q in range(S):
            _check_row(prio, q, s, w, k)
            assert np.flatnonzero(m[q]).tolist() == orc.kept_row_by_sorting(prio, q, s, w, k).tolist()
            assert held[q].tolist() == np.flatnonzero(m[q]).tolist()


@pytest.mark.parametrize("S,s,w,k", [(64, 4, 8, 16), (50, 0, 1, 7), (40, 3, 5, 0), (33, 2, 4, 100)])
def test_closed_forms(S, s, w, k):
    # priorities increasing in t: the newest eligible tokens win -> a sliding
    # window of w + k keys (plus sinks)
    inc = np.arange(S, dtype=np.float32)
    rank = orc.priority_rank(inc)
    tau = orc.thresholds_by_selection(rank[None], s, w, k)[0]
    m = orc.mask_rows(rank, tau, np.arange(S), s, w)
    for q in range(S):
        expect = [t for t in range(q + 1) if t < s or q - t < w + k]
        assert np.flatnonzero(m[q]).tolist() == expect
    # priorities decreasing in t: the oldest eligible tokens win -> {t < s + k} + window
    dec = -inc
    rank = orc.priority_rank(dec)
    tau = orc.thresholds_by_selection(rank[None], s, w, k)[0]
    m = orc.mask_rows(rank, tau, np.arange(S), s, w)
    for q in range(S):
        expect = [t for t in range(q + 1) if t < s + k and t <= q - w or t < s or q - t < w]
        assert np.flatnonzero(m[q]).tolist() == expect
    # k = 0: sinks + window only (StreamingLLM's rule)
    rng = np.random.default_rng(S)
    pr = rng.standard_normal(S).astype(np.float32)
    rank = orc.priority_rank(pr)
    tau0 = orc.thresholds_by_selection(rank[None], s, w, 0)[0]
    assert (tau0 == -1).all()
    m = orc.mask_rows(rank, tau0, np.arange(S), s, w)
    for q in range(S):
        assert np.flatnonzero(m[q]).tolist() == [t for t in range(q + 1) if t < s or q - t < w]
    # k >= S: plain causal
    taub = orc.thresholds_by_selection(rank[None], s, w, S)[0]
    assert (taub == orc.INT32_MAX).all()
    m = orc.mask_rows(rank, taub, np.arange(S), s, w)
    assert (m == np.tril(np.ones((S, S), dtype=bool))).all()


def test_cutoff_monotone_and_row_counts():
    rng = np.random.default_rng(5)
    S, s, w, k = 400, 4, 16, 32
    prio = rng.standard_normal((2, 3, S)).astype(np.float32)
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, k)
    first_full = s + w + k - 1       # first q with |E(q)| = k
    for i in range(2):
        for h in range(3):
            t = tau[i, h]
            assert (t[:first_full] == orc.INT32_MAX).all()
            assert np.all(np.diff(t[first_full:]) <= 0)
            m = orc.mask_rows(rank[i, h], t, np.arange(S), s, w)
            assert (m.sum(1) == np.minimum(np.arange(S) + 1, s + w + k)).all()
    # sampled rows agree with sorting route
    rows = [0, 19, 51, 52, 53, 200, 399]
    _, tau_sort = orc.thresholds_by_sorting(prio, s, w, k, rows=rows)
    assert (tau_sort == tau[..., rows]).all()


def test_decode_evicted_never_return_long_run():
    rng = np.random.default_rng(9)
    s, w, k, n = 3, 7, 11, 600
    table = rng.standard_normal(n).astype(np.float32).astype(np.float64)
    held, st = orc.decode_simulate(table, s, w, k, n)
    seen_evicted = set()
    prev = set()
    for p in range(n):
        cur = set(held[p].tolist())
        assert len(cur) == min(p + 1, s + w + k)
        seen_evicted |= (prev - cur)
        assert not (cur & seen_evicted)
        prev = cur
    # membership equals the prefill mask of the same priorities
    rank = orc.priority_rank(table.astype(np.float32))
    tau = orc.thresholds_by_selection(rank[None], s, w, k)[0]
    m = orc.mask_rows(rank, tau, np.arange(n), s, w)
    for p in range(0, n, 37):
        assert np.flatnonzero(m[p]).tolist() == held[p].tolist()
