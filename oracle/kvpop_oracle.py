"""Oracle for the KVpop fixed-budget KV-cache hot path (plain, slow, float64, CPU).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code,
header, table or helper with the HIP library under ``fixed_budget_sparse_amd/``,
and it never imports that package.

Sources (cited by page title; the section / equation named after each):
  [Notes]  "KVpop -- Key-Value Cache Compression with Predictive Online Pruning
           精读笔记" (reading notes, liuzhao09.github.io).  The only page with the
           method's formulas: B = s + w + k (§2.1), future mass m_t (§2.2),
           eligible set E(q) (§2.2), Eq. (8) (§2.3), Figure 2 (§2.3), sparse
           mask M_{q,t} and the rank cutoff tau_q (§2.3), delayed readout (§2.4).
  [Sum-zh] "技术摘要：KVpop — 基于预测性在线剪枝的键值（KV）缓存压缩"
           (gist.science summary): budget regions (§2.1), transposed pass
           returning LSE (§2.2), running threshold over static priorities (§2.4).
  [Trust]  "信任质量：KV-Cache淘汰中的强制权重" (forced weights in KV-cache
           eviction): Definition 2.1 (renormalised subset operator m_A) and the
           identity in the proof of Lemma 2.1.

Arithmetic is float64 (the pages fix no precision); integer outputs are exact.

Readings of points the pages leave open (each also listed in the design notes):
  R1 causality: the mask of [Notes] §2.3 has no t <= q term; keys after the
     query are never kept (the teacher is dense *causal* attention, [Notes] §2.2).
  R2 softmax scale defaults to 1/sqrt(D).
  R3 LSE is a natural log (Eq. (8) uses exp/log).
  R4 the target takes the caller's LSE; parity uses the dense causal LSE.
  R5 the target is the first term of Eq. (8) per query head: no -log N_t, no
     epsilon, no average over the query group; an empty range gives -inf.
  R6 priority order: higher priority first, ties to the lower token index;
     -0 == +0; NaN is treated as -inf.
  R7 tau_q = INT32_MAX when fewer than k tokens are eligible, -1 when k = 0.
  R8 query head h reads KV head h // (Hq / Hkv); priorities are per KV head.
  R9 decode order within a step: token p enters the window, then the token
     u = p - w leaving the window is kept (if fewer than k long-range tokens are
     held) or replaces the worst held long-range token iff its priority is
     strictly larger (worst = lowest priority, ties: highest position), else is
     dropped; then the step attends.
  R10 the target score's N_t is the number of future queries S - t - w; where
     there are none (t + w > S - 1) the future mass is 0 and the score is
     log(eps).
  R11 the decayed target score r(q, t) = r_t + floor((q - t)/n) log(gamma_h) is
     evaluated in float32 as one rounded product followed by one rounded sum
     (the labels are integer decisions taken on it, so both implementations
     take them in that precision); NaN scores count as -inf and -0 as +0.
  R12 teacher boundary labels: the teacher keeps the first min(k, |E(q)|)
     tokens of E(q) = [s, q - w] in the order (decayed score desc, index asc);
     t_bnd is the last kept token in that order (it may be t_new itself) and
     y = +1 if t_new = q - w is kept, -1 if not.  Without a newcomer
     (q - w < s) there is no label: y = 0, t_bnd = -1; with k = 0 nothing is
     kept: y = -1, t_bnd = -1.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

INT32_MAX = 2 ** 31 - 1


# --------------------------------------------------------------------------
# Priority order and rank  ([Notes] §2.3: rank(t) is the place of token t when
# tokens are ordered by their static priority; reading R6 for ties/NaN)
# --------------------------------------------------------------------------
def canonical_priority(p: np.ndarray) -> np.ndarray:
    """NaN -> -inf and -0 -> +0 (reading R6)."""
    p = np.array(p, dtype=np.float64, copy=True)
    p[np.isnan(p)] = -np.inf
    p[p == 0.0] = 0.0
    return p


def priority_rank(prio_row: np.ndarray) -> np.ndarray:
    """rank[t] = position of token t in the order (priority desc, index asc)."""
    p = canonical_priority(prio_row)
    S = p.shape[0]
    order = np.lexsort((np.arange(S), -p))   # primary key -p, then the index
    rank = np.empty(S, dtype=np.int64)
    rank[order] = np.arange(S)
    return rank


def priority_ranks(prio: np.ndarray) -> np.ndarray:
    """priority_rank over every leading index of prio[..., S]."""
    flat = prio.reshape(-1, prio.shape[-1])
    out = np.stack([priority_rank(r) for r in flat])
    return out.reshape(prio.shape)


# --------------------------------------------------------------------------
# Eligible set and long-range top-k  ([Notes] §2.2: E(q) = {t | s <= t <= q - w};
# [Notes] §2.1 / [Sum-zh] §2.1: k long-range slots among the older tokens)
# --------------------------------------------------------------------------
def eligible(q: int, s: int, w: int) -> range:
    return range(s, max(s, q - w + 1))


def kept_long_by_sorting(prio_row: np.ndarray, q: int, s: int, w: int, k: int) -> List[int]:
    """The long-range kept set at query q: sort E(q) by (priority desc, index
    asc) and take the first min(k, |E(q)|) tokens."""
    p = canonical_priority(prio_row)
    E = list(eligible(q, s, w))
    E.sort(key=lambda t: (-p[t], t))
    return sorted(E[:min(k, len(E))])


def tau_from_kept(rank_row: np.ndarray, kept_long: Sequence[int], n_eligible: int, k: int) -> int:
    """tau_q: the rank of the k-th best eligible token (reading R7 for the
    sentinels)."""
    if k == 0:
        return -1
    if n_eligible < k:
        return INT32_MAX
    return int(max(rank_row[t] for t in kept_long))


def thresholds_by_sorting(prio: np.ndarray, s: int, w: int, k: int,
                          rows: Optional[Sequence[int]] = None):
    """rank[..., S] and tau[..., rows] by sorting E(q) per row (slow: for tiny
    and sampled cases)."""
    rank = priority_ranks(prio)
    S = prio.shape[-1]
    rows = list(range(S)) if rows is None else list(rows)
    flat_p = prio.reshape(-1, S)
    flat_r = rank.reshape(-1, S)
    tau = np.empty((flat_p.shape[0], len(rows)), dtype=np.int64)
    for i in range(flat_p.shape[0]):
        for j, q in enumerate(rows):
            L = kept_long_by_sorting(flat_p[i], q, s, w, k)
            tau[i, j] = tau_from_kept(flat_r[i], L, len(eligible(q, s, w)), k)
    return rank, tau.reshape(prio.shape[:-1] + (len(rows),))


def thresholds_by_selection(rank: np.ndarray, s: int, w: int, k: int,
                            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """tau[..., rows]: the k-th smallest of rank[s .. q-w] (np.partition), a
    second route to the same cutoff."""
    S = rank.shape[-1]
    rows = list(range(S)) if rows is None else list(rows)
    flat = rank.reshape(-1, S)
    tau = np.empty((flat.shape[0], len(rows)), dtype=np.int64)
    for j, q in enumerate(rows):
        n = len(eligible(q, s, w))
        if k == 0:
            tau[:, j] = -1
        elif n < k:
            tau[:, j] = INT32_MAX
        else:
            seg = flat[:, s:q - w + 1]
            tau[:, j] = np.partition(seg, k - 1, axis=1)[:, k - 1]
    return tau.reshape(rank.shape[:-1] + (len(rows),))


# --------------------------------------------------------------------------
# Sparse mask  ([Notes] §2.3: M_{q,t} = 1[t<s] or 1[q-t<w] or (1[t in E(q)] and
# 1[rank(t) <= tau_q]); reading R1 adds t <= q)
# --------------------------------------------------------------------------
def mask_rows(rank_row: np.ndarray, tau_rows: np.ndarray, qs: np.ndarray, s: int, w: int) -> np.ndarray:
    """Boolean mask [len(qs), S] from rank and per-row cutoffs."""
    S = rank_row.shape[0]
    t = np.arange(S)[None, :]
    q = np.asarray(qs)[:, None]
    tau = np.asarray(tau_rows, dtype=np.int64)[:, None]
    in_e = (t >= s) & (t <= q - w)
    m = (t < s) | (q - t < w) | (in_e & (rank_row[None, :] <= tau))
    return m & (t <= q)


def kept_row_by_sorting(prio_row: np.ndarray, q: int, s: int, w: int, k: int) -> np.ndarray:
    """Sorted kept positions of row q: sinks, window, long-range top-k."""
    L = set(kept_long_by_sorting(prio_row, q, s, w, k))
    return np.array([t for t in range(q + 1) if t < s or q - t < w or t in L], dtype=np.int64)


# --------------------------------------------------------------------------
# Attention over a kept set  ([Notes] Figure 1 / §2.3: softmax over the retained
# set, LSE returned; [Trust] Definition 2.1: the renormalised subset mean m_A)
# --------------------------------------------------------------------------
def _attend(z: np.ndarray, v: np.ndarray, keep: np.ndarray):
    """z [n, S] logits, v [S, D], keep [n, S] -> O [n, D], LSE [n] (natural log)."""
    z = np.where(keep, z, -np.inf)
    mx = z.max(axis=1)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(z - mx_safe[:, None])
    den = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.log(den) + mx_safe
        o = (e @ v) / den[:, None]
    return o, lse


def default_scale(D: int, scale: float = 0.0) -> float:
    return scale if scale > 0 else 1.0 / math.sqrt(D)


def masked_attention(q, k, v, rank, tau, s, w, scale=0.0, rows=None, block=256):
    """Sparse attention forward with an explicit mask, row block by row block.

    q [b, Hq, S, D]; k, v [b, Hkv, S, D]; rank [b, Hkv, S]; tau [b, Hkv, S] (the
    cutoff of every row).  Returns O [b, Hq, n, D] and LSE [b, Hq, n] (float64)
    for ``rows`` (default: all S rows)."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    O = np.zeros((b, Hq, len(rows), D))
    LSE = np.zeros((b, Hq, len(rows)))
    for bi in range(b):
        for hq in range(Hq):
            h = hq // G                                   # reading R8
            K = k[bi, h].astype(np.float64)
            V = v[bi, h].astype(np.float64)
            for a in range(0, len(rows), block):
                qs = rows[a:a + block]
                keep = mask_rows(rank[bi, h], tau[bi, h, qs], qs, s, w)
                z = sc * (q[bi, hq, qs].astype(np.float64) @ K.T)
                O[bi, hq, a:a + block], LSE[bi, hq, a:a + block] = _attend(z, V, keep)
    return O, LSE


def masked_attention_backward(q, k, v, rank, tau, s, w, dout, scale=0.0, block=256):
    """Gradients of the sparse attention forward ([Notes] §2.3: the student's
    forward over the kept set; its backward is what training the sparse
    student with distillation needs, [Notes] §2.1) for an upstream gradient
    ``dout`` of O (the LSE output is taken as not differentiated).  Per query
    head and row i over the kept keys K_i, with P_it the renormalised
    probabilities and z_it = scale <q_i, k_t>:
        dV_t  = sum_i P_it dO_i                  (summed over the query group)
        dP_it = <dO_i, v_t>,  D_i = sum_t P_it dP_it
        dZ_it = P_it (dP_it - D_i)               (softmax Jacobian)
        dQ_i  = scale sum_t dZ_it k_t,  dK_t = scale sum_i dZ_it q_i (group sum).
    q, dout [b, Hq, S, D]; k, v [b, Hkv, S, D] -> dQ like q, dK and dV like k
    (float64)."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    dQ = np.zeros((b, Hq, S, D))
    dK = np.zeros((b, Hkv, S, D))
    dV = np.zeros((b, Hkv, S, D))
    for bi in range(b):
        for hq in range(Hq):
            h = hq // G                                   # reading R8
            K = k[bi, h].astype(np.float64)
            V = v[bi, h].astype(np.float64)
            for a in range(0, S, block):
                qs = np.arange(a, min(S, a + block))
                keep = mask_rows(rank[bi, h], tau[bi, h, qs], qs, s, w)
                Q = q[bi, hq, qs].astype(np.float64)
                dO = dout[bi, hq, qs].astype(np.float64)
                z = np.where(keep, sc * (Q @ K.T), -np.inf)
                mx = z.max(axis=1, keepdims=True)
                e = np.where(keep, np.exp(z - mx), 0.0)
                P = e / e.sum(axis=1, keepdims=True)
                dP = dO @ V.T
                Drow = (P * dP).sum(axis=1, keepdims=True)
                dZ = P * (dP - Drow)
                dQ[bi, hq, qs] = sc * (dZ @ K)
                dK[bi, h] += sc * (dZ.T @ Q)
                dV[bi, h] += P.T @ dO
    return dQ, dK, dV


def dense_causal_attention(q, k, v, scale=0.0, rows=None, block=256):
    """Dense causal attention (every key t <= q kept): the teacher."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    O = np.zeros((b, Hq, len(rows), D))
    LSE = np.zeros((b, Hq, len(rows)))
    t = np.arange(S)[None, :]
    for bi in range(b):
        for hq in range(Hq):
            h = hq // G
            K = k[bi, h].astype(np.float64)
            V = v[bi, h].astype(np.float64)
            for a in range(0, len(rows), block):
                qs = rows[a:a + block]
                keep = t <= qs[:, None]
                z = sc * (q[bi, hq, qs].astype(np.float64) @ K.T)
                O[bi, hq, a:a + block], LSE[bi, hq, a:a + block] = _attend(z, V, keep)
    return O, LSE


# --------------------------------------------------------------------------
# Future-attention target  ([Notes] §2.2: m_t = (1/N_t) sum_{d=t+w}^{S-1} A_{d,t};
# [Notes] §2.3 Eq. (8) and Figure 2: the transposed pass returns
# log sum_{d>=t+w} exp(l(d,t) - LSE_d), the first term of Eq. (8); reading R5)
# --------------------------------------------------------------------------
def future_target_colsum(q, k, lse, w, scale=0.0, block=256):
    """Column-sum form: P[d,t] = exp(l(d,t) - LSE_d) over the dense causal map,
    summed down each column over the future queries d >= t + w, then the log.

    q [b, Hq, S, D], k [b, Hkv, S, D], lse [b, Hq, S] -> target [b, Hq, S]."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    out = np.empty((b, Hq, S))
    t = np.arange(S)[None, :]
    for bi in range(b):
        for hq in range(Hq):
            K = k[bi, hq // G].astype(np.float64)
            col = np.zeros(S)
            for a in range(0, S, block):
                ds = np.arange(a, min(S, a + block))
                l = sc * (q[bi, hq, ds].astype(np.float64) @ K.T)
                P = np.exp(l - lse[bi, hq, ds].astype(np.float64)[:, None])
                future = t <= ds[:, None] - w        # d >= t + w (implies t <= d)
                col += np.where(future, P, 0.0).sum(axis=0)
            with np.errstate(divide="ignore"):
                out[bi, hq] = np.log(col)
    return out


def future_target_eq8(q, k, lse, w, scale=0.0, ts=None):
    """Row form of Eq. (8)'s first term: for each token t, a log-sum-exp over the
    future queries d in [t+w, S) of l(d,t) - LSE_d (the transposed pass of
    Figure 2, key t acting as the query).  Returns [b, Hq, len(ts)]."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    ts = np.arange(S) if ts is None else np.asarray(ts)
    out = np.empty((b, Hq, len(ts)))
    for bi in range(b):
        for hq in range(Hq):
            Qh = q[bi, hq].astype(np.float64)
            kv = k[bi, hq // G].astype(np.float64)
            L = lse[bi, hq].astype(np.float64)
            for j, t in enumerate(ts):
                d0 = t + w
                if d0 > S - 1:
                    out[bi, hq, j] = -np.inf
                    continue
                x = sc * (Qh[d0:] @ kv[t]) - L[d0:]
                m = x.max()
                out[bi, hq, j] = m + math.log(np.exp(x - m).sum())
    return out


def target_score(q, k, lse, w, eps, scale=0.0, block=256):
    """Target score per KV head ([Notes] §2.2): the future mass of query group g,
    m_t = (1/N_t) sum_{d=t+w}^{S-1} A_{d,t} with A the dense causal attention
    probabilities exp(l(d,t) - LSE_d) and N_t = S - t - w future queries, is
    averaged over the G query heads of the KV head and logged with eps:
    r_{h,t} = log(eps + (1/G) sum_g m_t^{(h,g)}).  Where N_t = 0 the mass is 0
    (reading R10).  q [b, Hq, S, D], k [b, Hkv, S, D], lse [b, Hq, S] ->
    r [b, Hkv, S] (float64)."""
    b, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    t = np.arange(S)
    n_t = S - t - w
    mass = np.zeros((b, Hkv, S))
    for bi in range(b):
        for hq in range(Hq):
            K = k[bi, hq // G].astype(np.float64)
            col = np.zeros(S)
            for a in range(0, S, block):
                ds = np.arange(a, min(S, a + block))
                A = np.exp(sc * (q[bi, hq, ds].astype(np.float64) @ K.T)
                           - lse[bi, hq, ds].astype(np.float64)[:, None])
                col += np.where(t[None, :] <= ds[:, None] - w, A, 0.0).sum(axis=0)
            with np.errstate(divide="ignore", invalid="ignore"):
                m = np.where(n_t > 0, col / np.maximum(n_t, 1), 0.0)
            mass[bi, hq // G] += m / G
    with np.errstate(divide="ignore"):
        return np.log(eps + mass)


# --------------------------------------------------------------------------
# Teacher boundary labels  ([Notes] §2.2: the decayed target score, the
# teacher's top-k over E(q), the boundary token t_bnd and the label y_{q,h};
# readings R11, R12)
# --------------------------------------------------------------------------
def decayed_scores(score_row: np.ndarray, q: int, n: int, log_gamma: float,
                   ts: np.ndarray) -> np.ndarray:
    """r(q, t) = r_t + floor((q - t) / n) * log(gamma) for the tokens ``ts``
    (float32 product, then float32 sum; NaN -> -inf, -0 -> +0; reading R11)."""
    age = ((q - ts) // n).astype(np.float32)
    r = score_row[ts].astype(np.float32) + age * np.float32(log_gamma)
    r = r.astype(np.float32)
    r[np.isnan(r)] = -np.inf
    r[r == 0] = 0.0
    return r


def teacher_kept(score_row: np.ndarray, q: int, s: int, w: int, k: int, n: int,
                 log_gamma: float) -> np.ndarray:
    """The teacher's kept long-range tokens at query q, best first: the first
    min(k, |E(q)|) tokens of E(q) = [s, q - w] by decayed score (descending),
    ties to the lower index (reading R12)."""
    ts = np.arange(s, q - w + 1)
    if len(ts) == 0 or k == 0:
        return ts[:0]
    r = decayed_scores(score_row, q, n, log_gamma, ts)
    order = np.lexsort((ts, -r.astype(np.float64)))   # primary key -r, then the index
    return ts[order[:min(k, len(ts))]]


def boundary_labels(score: np.ndarray, log_gamma: np.ndarray, n: int, s: int, w: int, k: int,
                    rows: Optional[Sequence[int]] = None):
    """Teacher boundary labels ([Notes] §2.2, reading R12).  score [b, Hkv, S]
    (the target score r^tgt), log_gamma [Hkv] -> (t_bnd, y), int32 [b, Hkv, S]:
    for every query q with a newcomer t_new = q - w >= s, t_bnd is the lowest
    ranked token the teacher keeps in E(q) and y = +1 / -1 as t_new is kept or
    not; other rows hold t_bnd = -1, y = 0 (k = 0: y = -1)."""
    b, H, S = score.shape
    t_bnd = np.full((b, H, S), -1, dtype=np.int32)
    y = np.zeros((b, H, S), dtype=np.int32)
    for bi in range(b):
        for h in range(H):
            for q in (range(S) if rows is None else rows):
                t_new = q - w
                if t_new < s:
                    continue
                kept = teacher_kept(score[bi, h], q, s, w, k, n, float(log_gamma[h]))
                if len(kept) == 0:
                    y[bi, h, q] = -1
                    continue
                t_bnd[bi, h, q] = kept[-1]
                y[bi, h, q] = 1 if t_new in set(kept.tolist()) else -1
    return t_bnd, y


# --------------------------------------------------------------------------
# Decode over a fixed-size cache  ([Notes] §2.3: inference keeps only the
# compact cache; [Notes] §2.4: token u = q - w is scored when it leaves the
# window; [Sum-zh] §2.1: sinks, protected window, k long-range slots;
# reading R9 for the order within a step and the replacement rule)
# --------------------------------------------------------------------------
class DecodeState:
    """Explicit sets of held positions for one (sequence, KV head)."""

    def __init__(self, s: int, w: int, k: int):
        self.s, self.w, self.k = s, w, k
        self.sinks: List[int] = []
        self.window: List[int] = []
        self.long: Dict[int, float] = {}      # position -> priority
        self.evicted: set = set()

    def step(self, p: int, prio_leaving: float) -> None:
        s, w, k = self.s, self.w, self.k
        if p < s:
            self.sinks.append(p)
        else:
            self.window.append(p)
        u = p - w
        if u >= s:
            assert self.window[0] == u
            self.window.pop(0)
            pu = prio_leaving
            if math.isnan(pu):
                pu = -math.inf
            if len(self.long) < k:
                self.long[u] = pu
            elif k == 0:
                self.evicted.add(u)
            else:
                # worst held long-range token: lowest priority, ties -> highest position
                m = min(self.long, key=lambda t: (self.long[t], -t))
                if pu > self.long[m]:
                    del self.long[m]
                    self.evicted.add(m)
                    self.long[u] = pu
                else:
                    self.evicted.add(u)

    def held(self) -> np.ndarray:
        return np.array(sorted(self.sinks + self.window + list(self.long)), dtype=np.int64)


def decode_simulate(prio_table: np.ndarray, s: int, w: int, k: int, n_steps: int,
                    record: Optional[Sequence[int]] = None):
    """Run steps p = 0..n_steps-1 for one (sequence, KV head).  prio_table[t] is the
    priority token t receives when it leaves the window.  Returns the held sets
    at the steps in ``record`` (default: every step) and the final state."""
    st = DecodeState(s, w, k)
    rec = set(range(n_steps)) if record is None else set(record)
    held = {}
    for p in range(n_steps):
        u = p - w
        st.step(p, float(prio_table[u]) if u >= s else float("nan"))
        if p in rec:
            held[p] = st.held()
    return held, st


def decode_attention(q_step, k_tokens, v_tokens, held, scale=0.0):
    """One decode step's output for one sequence.

    q_step [Hq, D]; k_tokens, v_tokens [Hkv, P, D] (token p's K/V is row p);
    held: list over KV heads of held positions.  Returns o [Hq, D], lse [Hq]."""
    Hq, D = q_step.shape
    Hkv = k_tokens.shape[0]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for hq in range(Hq):
        h = hq // G
        idx = np.asarray(held[h])
        z = sc * (k_tokens[h, idx].astype(np.float64) @ q_step[hq].astype(np.float64))
        keep = np.ones((1, len(idx)), dtype=bool)
        oo, ll = _attend(z[None, :], v_tokens[h, idx].astype(np.float64), keep)
        o[hq], lse[hq] = oo[0], ll[0]
    return o, lse
