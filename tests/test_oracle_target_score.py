"""Pins of the oracle's target score ([Notes] §2.2: future mass m_t averaged over
the query group and logged with eps) against closed forms and brute force."""
import math

import numpy as np

import oracle as orc


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_zero_queries_give_harmonic_mass():
    # Q = 0: every row is uniform over its causal prefix, A_{d,t} = 1/(d+1), so
    # m_t = (H_S - H_{t+w}) / (S - t - w) for every head.
    b, hq, hkv, S, D, w, eps = 1, 4, 2, 40, 8, 3, 1e-6
    q = np.zeros((b, hq, S, D))
    k = _rand((b, hkv, S, D), 1)
    lse = np.log(np.arange(1, S + 1, dtype=np.float64))[None, None, :].repeat(hq, 1)
    r = orc.target_score(q, k, lse, w, eps)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, S + 1))])
    for t in range(S):
        n = S - t - w
        want = math.log(eps + ((H[S] - H[t + w]) / n if n > 0 else 0.0))
        assert np.allclose(r[0, :, t], want, rtol=0, atol=1e-12), t


def test_no_future_queries_give_log_eps():
    b, hq, hkv, S, D, w = 1, 2, 1, 16, 4, 5
    q, k = _rand((b, hq, S, D), 2), _rand((b, hkv, S, D), 3)
    _, lse = orc.dense_causal_attention(q, k, k)
    for eps in (0.5, 1e-3):
        r = orc.target_score(q, k, lse, w, eps)
        assert np.allclose(r[0, 0, S - w:], math.log(eps))
    r0 = orc.target_score(q, k, lse, w, 0.0)
    assert np.isneginf(r0[0, 0, S - w:]).all() and np.isfinite(r0[0, 0, :S - w]).all()


def test_identical_heads_reduce_to_one_head():
    b, hkv, S, D, w, eps = 1, 1, 30, 8, 2, 1e-4
    q1, k = _rand((b, 1, S, D), 4), _rand((b, hkv, S, D), 5)
    _, lse1 = orc.dense_causal_attention(q1, k, k)
    q3 = np.repeat(q1, 3, axis=1)
    lse3 = np.repeat(lse1, 3, axis=1)
    assert np.allclose(orc.target_score(q3, k, lse3, w, eps), orc.target_score(q1, k, lse1, w, eps))


def test_matches_column_sum_target_shifted_by_ln_n():
    # exp(target_g) is the column sum of A; the score is its mean over the group
    # divided by N_t (two routes through different code of the oracle).
    b, hq, hkv, S, D, w, eps = 1, 6, 2, 50, 8, 4, 1e-3
    q, k = _rand((b, hq, S, D), 6), _rand((b, hkv, S, D), 7)
    _, lse = orc.dense_causal_attention(q, k, k)
    T = orc.future_target_eq8(q, k, lse, w)
    n = S - np.arange(S) - w
    G = hq // hkv
    with np.errstate(divide="ignore"):
        m = np.where(n > 0, np.exp(T - np.log(np.maximum(n, 1))), 0.0)
        want = np.log(eps + m.reshape(b, hkv, G, S).mean(axis=2))
    got = orc.target_score(q, k, lse, w, eps)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny():
    b, hq, hkv, S, D, w, eps = 1, 2, 1, 7, 3, 2, 0.01
    q, k = _rand((b, hq, S, D), 8), _rand((b, hkv, S, D), 9)
    sc = 1 / math.sqrt(D)
    A = np.zeros((hq, S, S))
    for h in range(hq):
        for d in range(S):
            z = [sc * float(np.dot(q[0, h, d], k[0, 0, t])) for t in range(d + 1)]
            mx = max(z)
            den = sum(math.exp(x - mx) for x in z)
            for t in range(d + 1):
                A[h, d, t] = math.exp(z[t] - mx) / den
    _, lse = orc.dense_causal_attention(q, k, k)
    got = orc.target_score(q, k, lse, w, eps)
    for t in range(S):
        ds = range(t + w, S)
        mass = sum(sum(A[h, d, t] for d in ds) / len(ds) for h in range(hq)) / hq if len(ds) else 0.0
        assert abs(got[0, 0, t] - math.log(eps + mass)) < 1e-12, t
