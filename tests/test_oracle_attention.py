"""Pins for the oracle's masked forward, dense LSE, future target and decode output.

Every check compares the oracle with something it does not compute itself:
library attention (torch's scaled_dot_product_attention, scipy's logsumexp),
closed forms (zero queries, constant values, harmonic sums), exact identities
(the renormalised-subset identity from the proof of Lemma 2.1 of "信任质量：
KV-Cache淘汰中的强制权重"; rows summing to one; the w = 0 column-mass total),
and brute-force pure-Python loops on tiny inputs.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc


def _inputs(b, Hq, Hkv, S, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, Hq, S, D)).astype(np.float32)
    k = rng.standard_normal((b, Hkv, S, D)).astype(np.float32)
    k[:, :, :4] *= 4
    v = rng.standard_normal((b, Hkv, S, D)).astype(np.float32)
    prio = rng.standard_normal((b, Hkv, S)).astype(np.float32)
    return q, k, v, prio


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch library attention in float64 with GQA head sharing."""
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    tk = tk.repeat_interleave(G, dim=1)
    tv = tv.repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, is_causal=causal, scale=scale).numpy()


def test_dense_special_case_matches_library():
    # k >= S keeps every causal key: textbook causal attention
    q, k, v, prio = _inputs(2, 4, 2, 96, 16, 1)
    s, w, kk = 3, 5, 96
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, kk)
    O, LSE = orc.masked_attention(q, k, v, rank, tau, s, w)
    ref = _sdpa(q, k, v, causal=True)
    assert np.abs(O - ref).max() < 1e-12
    Od, LSEd = orc.dense_causal_attention(q, k, v)
    assert np.abs(Od - ref).max() < 1e-12
    assert np.abs(LSE - LSEd).max() < 1e-12
    # LSE against a library log-sum-exp of the causal logits
    sc = 1 / math.sqrt(16)
    for bi in range(2):
        for hq in range(4):
            z = sc * q[bi, hq].astype(np.float64) @ k[bi, hq // 2].astype(np.float64).T
            z[np.triu_indices(96, 1)] = -np.inf
            assert np.abs(scipy.special.logsumexp(z, axis=1) - LSEd[bi, hq]).max() < 1e-12


def test_sliding_window_special_case_matches_library():
    # s = k = 0: textbook sliding-window attention over the w newest keys
    q, k, v, prio = _inputs(1, 2, 1, 80, 8, 2)
    w = 7
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, 0, w, 0)
    O, _ = orc.masked_attention(q, k, v, rank, tau, 0, w)
    ones = torch.ones(80, 80, dtype=torch.bool)
    band = (torch.tril(ones) & ~torch.tril(ones, diagonal=-w)).numpy()
    ref = _sdpa(q, k, v, mask=band)
    assert np.abs(O - ref).max() < 1e-12


def test_sparse_mask_matches_library_with_explicit_mask():
    q, k, v, prio = _inputs(1, 4, 2, 70, 8, 3)
    s, w, kk = 2, 6, 9
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, kk)
    O, _ = orc.masked_attention(q, k, v, rank, tau, s, w, scale=0.3)
    for h in range(2):
        # the mask built by sorting, row by row, independent of rank/tau
        mask = np.zeros((70, 70), dtype=bool)
        for qq in range(70):
            mask[qq, orc.kept_row_by_sorting(prio[0, h], qq, s, w, kk)] = True
        ref = _sdpa(q[:, 2 * h:2 * h + 2], k[:, h:h + 1], v[:, h:h + 1], mask=mask, scale=0.3)
        assert np.abs(O[:, 2 * h:2 * h + 2] - ref).max() < 1e-12


def test_zero_query_closed_form():
    # Q = 0: every kept logit is 0 -> LSE_q = ln min(q+1, B) and O_q = mean of kept V rows
    q, k, v, prio = _inputs(1, 2, 1, 120, 8, 4)
    q[:] = 0
    s, w, kk = 4, 9, 13
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, kk)
    O, LSE = orc.masked_attention(q, k, v, rank, tau, s, w)
    n = np.minimum(np.arange(120) + 1, s + w + kk)
    assert np.abs(LSE[0, 0] - np.log(n)).max() < 1e-12
    for qq in (0, 5, 30, 119):
        kept = orc.kept_row_by_sorting(prio[0, 0], qq, s, w, kk)
        assert np.abs(O[0, 1, qq] - v[0, 0, kept].astype(np.float64).mean(0)).max() < 1e-12


def test_constant_values_and_rows_sum_to_one():
    q, k, v, prio = _inputs(1, 4, 2, 64, 8, 5)
    v[:] = 1.75
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, 2, 4, 5)
    O, _ = orc.masked_attention(q, k, v, rank, tau, 2, 4)
    assert np.abs(O - 1.75).max() < 1e-12


def test_renormalised_subset_identity():
    """Proof of Lemma 2.1 ([Trust]): mu - m_A = sum_{j not in A} p_j (v_j - mu) / p(A),
    with p the dense causal row, mu the dense output and m_A the sparse output;
    also LSE_sparse = LSE_dense + ln p(A) and the bound |mu - m_A| <= D pbar/(1-pbar)."""
    q, k, v, prio = _inputs(1, 2, 1, 90, 8, 6)
    s, w, kk = 2, 5, 6
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, kk)
    O, LSE = orc.masked_attention(q, k, v, rank, tau, s, w)
    mu = _sdpa(q, k, v, causal=True)
    sc = 1 / math.sqrt(8)
    for hq in range(2):
        z = sc * q[0, hq].astype(np.float64) @ k[0, 0].astype(np.float64).T
        z[np.triu_indices(90, 1)] = -np.inf
        P = scipy.special.softmax(z, axis=1)
        lse_d = scipy.special.logsumexp(z, axis=1)
        V = v[0, 0].astype(np.float64)
        for qq in range(90):
            A = orc.kept_row_by_sorting(prio[0, 0], qq, s, w, kk)
            drop = np.setdiff1d(np.arange(qq + 1), A)
            pA = P[qq, A].sum()
            lhs = mu[0, hq, qq] - O[0, hq, qq]
            rhs = (P[qq, drop, None] * (V[drop] - mu[0, hq, qq])).sum(0) / pA
            assert np.abs(lhs - rhs).max() < 1e-11 / pA
            assert abs(LSE[0, hq, qq] - (lse_d[qq] + math.log(pA))) < 1e-11
            if len(drop):
                Dmax = np.linalg.norm(V[:qq + 1] - mu[0, hq, qq], axis=1).max()
                pbar = 1 - pA
                assert np.linalg.norm(lhs) <= Dmax * pbar / (1 - pbar) + 1e-12


def test_gqa_head_map_matches_library_sharing():
    q, k, v, prio = _inputs(1, 6, 2, 40, 8, 7)
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, 0, 1, 40)
    O, _ = orc.masked_attention(q, k, v, rank, tau, 0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64)), is_causal=True, enable_gqa=True).numpy()
    assert np.abs(O - ref).max() < 1e-12


# ---------------------------------------------------------------- targets
def _dense_lse(q, k):
    return orc.dense_causal_attention(q, k, k)[1]


def test_target_w0_total_mass_is_S():
    # with w = 0 every causal pair is summed; dense rows sum to one -> sum_t exp(target_t) = S
    q, k, _, _ = _inputs(2, 4, 2, 77, 16, 8)
    lse = _dense_lse(q, k)
    T = orc.future_target_colsum(q, k, lse, 0)
    assert np.abs(np.exp(T).sum(-1) - 77).max() < 1e-10


def test_target_zero_query_harmonic_closed_form():
    # Q = 0: p(d,t) = 1/(d+1) -> target_t = ln(H_S - H_{t+w})
    q, k, _, _ = _inputs(1, 2, 1, 60, 8, 9)
    q[:] = 0
    w = 5
    lse = _dense_lse(q, k)
    T = orc.future_target_colsum(q, k, lse, w)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, 61))])
    for t in range(60):
        want = math.log(H[60] - H[t + w]) if t + w <= 59 else -math.inf
        assert T[0, 0, t] == pytest.approx(want, abs=1e-12) if math.isfinite(want) else T[0, 0, t] == -np.inf


def test_target_single_term_and_empty_ranges():
    q, k, _, _ = _inputs(1, 2, 1, 50, 8, 10)
    w = 6
    lse = _dense_lse(q, k)
    T = orc.future_target_colsum(q, k, lse, w)
    t = 50 - 1 - w                      # only d = S-1 contributes
    sc = 1 / math.sqrt(8)
    z = sc * q[0, 1, 49].astype(np.float64) @ k[0, 0].astype(np.float64).T
    logp = z[t] - scipy.special.logsumexp(z[:50])
    assert T[0, 1, t] == pytest.approx(logp, abs=1e-12)
    assert np.all(T[0, :, 50 - w:] == -np.inf)
    T2 = orc.future_target_colsum(q, k, lse, 50)
    assert np.all(T2 == -np.inf)


def test_target_colsum_equals_eq8_and_bruteforce():
    q, k, _, _ = _inputs(1, 4, 2, 33, 8, 12)
    w = 3
    lse = _dense_lse(q, k)
    T = orc.future_target_colsum(q, k, lse, w)
    T8 = orc.future_target_eq8(q, k, lse, w)
    fin = np.isfinite(T)
    assert (fin == np.isfinite(T8)).all()
    assert np.abs(T[fin] - T8[fin]).max() < 1e-12
    # pure-python brute force on one head: sum over the dense map column
    sc = 1 / math.sqrt(8)
    hq, S = 3, 33
    Qh, Kh = q[0, hq].astype(float), k[0, 1].astype(float)
    for t in range(S):
        acc = 0.0
        for d in range(S):
            if d >= t + w:
                logit = sc * sum(Qh[d, i] * Kh[t, i] for i in range(8))
                den = sum(math.exp(sc * sum(Qh[d, i] * Kh[j, i] for i in range(8))) for j in range(d + 1))
                acc += math.exp(logit) / den
        want = math.log(acc) if acc > 0 else -math.inf
        if math.isfinite(want):
            assert T[0, hq, t] == pytest.approx(want, abs=1e-11)
        else:
            assert T[0, hq, t] == -np.inf


# ---------------------------------------------------------------- decode
def test_decode_output_equals_prefill_row():
    rng = np.random.default_rng(13)
    Hq, Hkv, D, s, w, kk, n = 4, 2, 8, 2, 5, 6, 60
    ks = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    vs = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    qs = rng.standard_normal((n, Hq, D)).astype(np.float32)
    prio = rng.standard_normal((Hkv, n)).astype(np.float32)
    states = [orc.DecodeState(s, w, kk) for _ in range(Hkv)]
    rank = orc.priority_ranks(prio[None])
    tau = orc.thresholds_by_selection(rank, s, w, kk)
    # prefill rows computed with every row's own query
    for p in range(n):
        for h in range(Hkv):
            u = p - w
            states[h].step(p, float(prio[h, u]) if u >= s else float("nan"))
        held = [st.held() for st in states]
        o, lse = orc.decode_attention(qs[p], ks, vs, held)
        qfull = np.zeros((1, Hq, n, D), dtype=np.float32)
        qfull[0, :, p] = qs[p]
        O, L = orc.masked_attention(qfull, ks[None], vs[None], rank, tau, s, w, rows=[p])
        assert np.abs(o - O[0, :, 0]).max() < 1e-12
        assert np.abs(lse - L[0, :, 0]).max() < 1e-12
