"""Pins of the oracle's teacher boundary labels ([Notes] §2.2: decayed target
score, the teacher's top-k over E(q), boundary token t_bnd and label y; readings
R11, R12): hand-worked examples, reductions to the static-priority cutoffs of
[Notes] §2.3 (no decay, and n = 1 with exact arithmetic, where the floor decay
is a linear one), and a pairwise brute force of the selection."""
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_labels.txt")


def _cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line == "case":
            cur = {}
        elif line == "end":
            cases.append(cur)
        else:
            key, *vals = line.split()
            cur[key] = vals
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "S{}k{}n{}".format(c["S"][0], c["k"][0], c["n"][0]))
def test_hand_worked(case):
    S, s, w, k, n = (int(case[x][0]) for x in ("S", "s", "w", "k", "n"))
    lg = float(case["log_gamma"][0])
    score = np.array([float(v) for v in case["score"]], dtype=np.float32).reshape(1, 1, S)
    t_bnd, y = orc.boundary_labels(score, np.array([lg], np.float32), n, s, w, k)
    assert t_bnd[0, 0].tolist() == [int(v) for v in case["t_bnd"]]
    assert y[0, 0].tolist() == [int(v) for v in case["y"]]


def _static_labels(prio, s, w, k):
    """Labels implied by the static-priority cutoffs of [Notes] §2.3: the kept
    long-range tokens are those of E(q) with rank <= tau_q, so t_new is kept iff
    rank(t_new) <= tau_q and the last kept token is the one ranked tau_q (the
    worst-ranked eligible token while fewer than k are eligible)."""
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, k)
    b, H, S = prio.shape
    t_bnd = np.full((b, H, S), -1, np.int32)
    y = np.zeros((b, H, S), np.int32)
    for bi in range(b):
        for h in range(H):
            r = rank[bi, h]
            inv = np.argsort(r)
            for q in range(S):
                t_new = q - w
                if t_new < s:
                    continue
                if k == 0:
                    y[bi, h, q] = -1
                    continue
                T = int(tau[bi, h, q])
                E = np.arange(s, t_new + 1)
                t_bnd[bi, h, q] = E[np.argmax(r[E])] if T == orc.INT32_MAX else inv[T]
                y[bi, h, q] = 1 if r[t_new] <= T else -1
    return t_bnd, y


def _scores(shape, seed, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if ties:
        x = np.round(x * 2).astype(np.float32) / 2
        x.flat[rng.integers(0, x.size, max(1, x.size // 25))] = np.nan
        x.flat[rng.integers(0, x.size, max(1, x.size // 40))] = -np.inf
        x.flat[rng.integers(0, x.size, max(1, x.size // 40))] = np.inf
        x[x == 0] = -0.0
    return x


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("s,w,k", [(2, 5, 7), (0, 1, 1), (3, 4, 0), (1, 3, 60)])
def test_no_decay_is_the_static_cutoff(ties, s, w, k):
    # log(gamma) = 0, and a decay step longer than the sequence, both leave the
    # order static: the labels follow from rank and tau_q.
    score = _scores((2, 2, 70), 11, ties)
    want = _static_labels(score, s, w, k)
    for lg, n in ((np.zeros(2, np.float32), 3), (np.array([-0.7, -2.5], np.float32), 71)):
        got = orc.boundary_labels(score, lg, n, s, w, k)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), (lg, n)


@pytest.mark.parametrize("s,w,k", [(2, 3, 5), (0, 2, 1), (4, 1, 9)])
def test_unit_step_is_a_linear_decay(s, w, k):
    # n = 1: floor((q - t)/1) = q - t, so r(q, t) = (r_t - t log g) + q log g and
    # the order is the static one of r_t - t log g.  Integer scores and
    # log g = -1 keep every value exact in float32.
    rng = np.random.default_rng(5)
    score = rng.integers(-40, 40, (1, 2, 80)).astype(np.float32)
    got = orc.boundary_labels(score, np.array([-1.0, -1.0], np.float32), 1, s, w, k)
    prio = score + np.arange(80, dtype=np.float32)
    want = _static_labels(prio, s, w, k)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


@pytest.mark.parametrize("seed,n,lg,s,w,k,ties", [
    (1, 3, -0.4, 2, 3, 4, False), (2, 1, -1.3, 0, 1, 2, True), (3, 5, -0.05, 1, 4, 10, True),
    (4, 2, -3.0, 3, 2, 1, False), (5, 7, -0.9, 0, 6, 30, True)])
def test_pairwise_brute_force(seed, n, lg, s, w, k, ties):
    # t_new is kept iff fewer than k eligible tokens precede it; t_bnd is the
    # eligible token with exactly min(k, |E|) - 1 predecessors, where u
    # precedes t iff r(q,u) > r(q,t) or (equal and u < t).
    S = 36
    score = _scores((1, 1, S), seed, ties)
    t_bnd, y = orc.boundary_labels(score, np.array([lg], np.float32), n, s, w, k)
    for q in range(S):
        t_new = q - w
        if t_new < s:
            assert y[0, 0, q] == 0 and t_bnd[0, 0, q] == -1
            continue
        E = list(range(s, t_new + 1))
        r = {}
        for t in E:
            v = np.float32(score[0, 0, t]) + np.float32((q - t) // n) * np.float32(lg)
            r[t] = -np.inf if np.isnan(v) else float(v)

        def before(u, t):
            return r[u] > r[t] or (r[u] == r[t] and u < t)

        preds = {t: sum(before(u, t) for u in E if u != t) for t in E}
        if k == 0:
            assert y[0, 0, q] == -1 and t_bnd[0, 0, q] == -1
            continue
        assert y[0, 0, q] == (1 if preds[t_new] < k else -1), q
        last = [t for t in E if preds[t] == min(k, len(E)) - 1]
        assert len(last) == 1 and t_bnd[0, 0, q] == last[0], q


def test_label_invariants():
    score = _scores((1, 3, 120), 9, True)
    lg = np.array([-0.2, -1.0, -0.01], np.float32)
    s, w, k, n = 4, 8, 20, 6
    t_bnd, y = orc.boundary_labels(score, lg, n, s, w, k)
    for h in range(3):
        for q in range(120):
            t_new = q - w
            if t_new < s:
                continue
            kept = orc.teacher_kept(score[0, h], q, s, w, k, n, float(lg[h]))
            assert len(kept) == min(k, t_new - s + 1)
            assert s <= t_bnd[0, h, q] <= t_new and t_bnd[0, h, q] == kept[-1]
            # while fewer than k are eligible every one is kept
            if t_new - s + 1 <= k:
                assert y[0, h, q] == 1
