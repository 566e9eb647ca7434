"""GPU parity of the calls beyond the hot path's core: the target score per KV
head and the study of a sparse-LSE target ([Notes] §2.2, §2.3), and the
prefill -> decode cache handoff ([Notes] §2.3).  Integer outputs bit-exact,
floats within the stated tolerances; every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import fixed_budget_sparse_amd as kv
import oracle as orc
from gpu_util import BF16_U, BWD_TOL, TOL, announce, device, host, to_dev

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale_keys=False):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    if scale_keys:
        x[..., :4, :] *= 4
    return x


def _bf16(x):
    from workloads import round_to_bf16
    return round_to_bf16(x)


# ---------------------------------------------------------------- target score
SCORE_CASES = [
    # b, Hq, Hkv, S, D, w, eps
    (1, 8, 2, 640, 128, 32, 1e-6),
    (2, 4, 2, 300, 64, 0, 1e-3),
    (1, 6, 2, 257, 128, 17, 0.0),      # eps = 0: -inf where no future query
    (1, 4, 4, 200, 128, 300, 1e-6),    # w >= S: log(eps) everywhere
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: "b{}q{}kv{}S{}D{}w{}eps{}".format(*c))
def test_target_score_parity(case):
    b, hq, hkv, S, D, w, eps = case
    announce(f"target_score {case}")
    q = _bf16(_rand((b, hq, S, D), 51))
    k = _bf16(_rand((b, hkv, S, D), 52, scale_keys=True))
    _, LSE = orc.dense_causal_attention(q, k, k)
    L32 = LSE.astype(np.float32)
    R = orc.target_score(q, k, L32.astype(np.float64), w, eps)
    # the score kernel alone, on the oracle's targets
    T = orc.future_target_colsum(q, k, L32.astype(np.float64), w)
    r1 = host(kv.target_score(to_dev(T.astype(np.float32)), hkv, w, eps))
    fin = np.isfinite(R)
    assert np.array_equal(np.isneginf(r1), np.isneginf(R))
    assert np.abs(r1[fin] - R[fin]).max() <= 1e-5
    # the whole chain: GPU target, then GPU score
    tgt = kv.future_target(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(L32), w)
    r2 = host(kv.target_score(tgt, hkv, w, eps))
    assert np.array_equal(np.isneginf(r2), np.isneginf(R))
    sel = fin & (R > -20)
    if sel.any():
        assert np.abs(r2[sel] - R[sel]).max() <= TOL["bf16"]["tgt"], np.abs(r2[sel] - R[sel]).max()


def test_target_with_sparse_lse():
    """The approximate target of [Sum-zh] §2.2 / [Notes] §2.3: the transposed
    pass driven by the sparse forward's LSE instead of the teacher's.  It
    matches the oracle fed with the oracle's sparse LSE, and it is never below
    the exact target (a sparse LSE is at most the dense one)."""
    device()
    b, hq, hkv, S, D, s, w, k = 1, 8, 2, 700, 128, 4, 40, 100
    announce("target with sparse LSE")
    q = _bf16(_rand((b, hq, S, D), 61))
    kk = _bf16(_rand((b, hkv, S, D), 62, scale_keys=True))
    v = _bf16(_rand((b, hkv, S, D), 63))
    prio = _rand((b, hkv, S), 64)
    td = torch.bfloat16
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    _, lse_sparse = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s,
                                       w, k, out_dtype=torch.float32)
    tgt_sparse = host(kv.future_target(to_dev(q, td), to_dev(kk, td), lse_sparse, w))
    rank_o = orc.priority_ranks(prio)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    _, LS = orc.masked_attention(q, kk, v, rank_o, tau_o, s, w)
    T_s = orc.future_target_colsum(q, kk, LS.astype(np.float32).astype(np.float64), w)
    _, LD = orc.dense_causal_attention(q, kk, kk)
    T_d = orc.future_target_colsum(q, kk, LD.astype(np.float32).astype(np.float64), w)
    sel = np.isfinite(T_s) & (T_s > -20)
    assert np.abs(tgt_sparse[sel] - T_s[sel]).max() <= TOL["bf16"]["tgt"]
    fin = np.isfinite(T_d)
    assert (T_s[fin] >= T_d[fin] - 1e-9).all()
    assert (tgt_sparse[fin] >= T_d[fin] - TOL["bf16"]["tgt"]).all()


RESCALE_CASES = [
    # b, Hq, Hkv, S, D, w, lse kind, dtype
    (1, 4, 2, 600, 128, 20, "minus100", "bf16"),   # every exponent up to ~+100 nats: overflow
    (1, 4, 2, 600, 128, 20, "plus120", "bf16"),    # every term below e^-100: underflow
    (1, 4, 1, 900, 128, 7, "early", "bf16"),       # only the first tile's rows overflow
    (1, 2, 1, 300, 64, 5, "minus100", "f32"),      # float32 inputs, D = 64
    (1, 4, 2, 520, 64, 0, "plus120", "bf16"),      # w = 0, D = 64
]


@pytest.mark.parametrize("case", RESCALE_CASES, ids=lambda c: "b{}q{}kv{}S{}D{}w{}-{}-{}".format(*c))
def test_target_any_lse(case):
    """The target for an LSE that does not bound the row's logits (or sits far
    above them): the max-free sum would overflow (or underflow), so those tiles
    take the running-maximum pass; every finite target matches the oracle
    (float64, the same LSE), and no non-empty range gives +-inf."""
    b, hq, hkv, S, D, w, kind, dt = case
    announce(f"target any lse {case}")
    device()
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    q = _rand((b, hq, S, D), 111)
    kk = _rand((b, hkv, S, D), 112, scale_keys=True)
    if dt == "bf16":
        q, kk = _bf16(q), _bf16(kk)
    _, LD = orc.dense_causal_attention(q, kk, kk)
    L = LD.copy()
    if kind == "minus100":
        L -= 100.0
    elif kind == "plus120":
        L += 120.0
    elif kind == "early":
        L[..., :200] -= 100.0        # queries d < 200: only tokens t < 200 - w see them
    L32 = L.astype(np.float32)
    tgt = host(kv.future_target(to_dev(q, td), to_dev(kk, td), to_dev(L32), w))
    T = orc.future_target_colsum(q, kk, L32.astype(np.float64), w)
    assert np.array_equal(np.isneginf(tg := tgt), np.isneginf(T))
    assert not np.isposinf(tg).any() and not np.isnan(tg).any()
    fin = np.isfinite(T)
    tol = TOL[dt]["tgt"]
    assert np.abs(tg[fin] - T[fin]).max() <= tol, np.abs(tg[fin] - T[fin]).max()
    # the score stays finite and exact for targets far above ln N_t
    if kind != "plus120":
        R = orc.target_score(q, kk, L32.astype(np.float64), w, 1e-6)
        r = host(kv.target_score(to_dev(tg.astype(np.float32)), hkv, w, 1e-6))
        assert np.array_equal(np.isfinite(r), np.isfinite(R))
        f = np.isfinite(R)
        assert np.abs(r[f] - R[f]).max() <= tol, np.abs(r[f] - R[f]).max()


def test_target_planted_dropped_key():
    """A key dropped by the sparse mask whose logit exceeds the sparse LSE of
    later queries by about 150 nats ([Notes] §2.3: the sparse LSE approximates
    the dense one and must be checked): the target driven by that sparse LSE
    matches the oracle fed the same LSE, with no overflow."""
    device()
    b, hq, hkv, S, D, s, w, k = 1, 4, 1, 400, 128, 2, 8, 20
    announce("target with a planted dropped key")
    q = _rand((b, hq, S, D), 121)
    kk = _rand((b, hkv, S, D), 122)
    v = _rand((b, hkv, S, D), 123)
    t_star = 50
    prio = _rand((b, hkv, S), 124)
    prio[..., t_star] = -1e9                                    # never kept once it leaves the window
    q, v = _bf16(q), _bf16(v)
    # aligned with the last query of head 0: a logit of about 200 there
    u = q[0, 0, S - 1]
    kk[0, 0, t_star] = u * (200.0 * np.sqrt(D) / float(u @ u))
    kk = _bf16(kk)
    td = torch.bfloat16
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    _, lse_sparse = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s,
                                       w, k, out_dtype=torch.float32)
    L = host(lse_sparse)
    logit = float(q[0, 0, S - 1].astype(np.float64) @ kk[0, 0, t_star]) / np.sqrt(D)
    assert logit - L[0, 0, S - 1] > 88.0                       # beyond float32's exp range
    tgt = host(kv.future_target(to_dev(q, td), to_dev(kk, td), lse_sparse, w))
    T = orc.future_target_colsum(q, kk, L.astype(np.float64), w)
    assert np.isfinite(tgt[..., t_star]).all() and tgt[0, 0, t_star] > 80
    assert np.array_equal(np.isneginf(tgt), np.isneginf(T))
    fin = np.isfinite(T)
    assert np.abs(tgt[fin] - T[fin]).max() <= TOL["bf16"]["tgt"], np.abs(tgt[fin] - T[fin]).max()


# ---------------------------------------------------------------- handoff
HANDOFF_CASES = [
    # nseq, Hkv, D, S, s, w, k, prio kind, dtype
    (2, 2, 128, 300, 4, 16, 40, "normal", "bf16"),     # full cache (S > Bc)
    (2, 1, 128, 30, 4, 16, 40, "normal", "bf16"),      # partial fill (S < Bc)
    (1, 2, 64, 200, 3, 9, 20, "ties", "f32"),          # ties, NaN, +-inf; float32 cache
    (1, 2, 128, 100, 2, 7, 0, "normal", "bf16"),       # k = 0: sinks + window
    (1, 1, 128, 20, 2, 40, 10, "normal", "bf16"),      # w > S: no eligible token
    (1, 2, 128, 1, 1, 1, 5, "normal", "bf16"),         # a one-token prompt
    (1, 2, 128, 1500, 4, 100, 600, "normal", "bf16"),  # B = 704: two slot blocks, long range crosses
    (2, 1, 64, 600, 5, 300, 900, "ties", "bf16"),      # B = 1205, partial fill over three blocks
    (1, 1, 128, 2000, 600, 64, 300, "normal", "f32"),  # sinks fill the first block and more
]


def _prio(kind, shape, seed):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(shape).astype(np.float32)
    if kind == "ties":
        p = np.round(p * 2).astype(np.float32)
        p.flat[rng.integers(0, p.size, max(1, p.size // 30))] = np.nan
        p.flat[rng.integers(0, p.size, max(1, p.size // 50))] = np.inf
        p.flat[rng.integers(0, p.size, max(1, p.size // 50))] = -np.inf
        p[p == 0] = -0.0
    return p


@pytest.mark.parametrize("case", HANDOFF_CASES, ids=lambda c: "n{}kv{}D{}S{}s{}w{}k{}-{}-{}".format(*c))
def test_cache_from_prefill(case):
    nseq, hkv, D, S, s, w, k, kind, dt = case
    announce(f"cache_from_prefill {case}")
    dev = device()
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    Bc = s + w + k
    prio = _prio(kind, (nseq, hkv, S), 71)
    K = _rand((nseq, hkv, S, D), 72)
    V = _rand((nseq, hkv, S, D), 73)
    if dt == "bf16":
        K, V = _bf16(K), _bf16(V)
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    cache = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    cache.slot_pos.fill_(12345)            # every slot must be rewritten
    kv.cache_from_prefill(cache, to_dev(K, td), to_dev(V, td), to_dev(prio), rank, tau, s, w, k)
    torch.cuda.synchronize()
    sp, sprio, ring = host(cache.slot_pos), host(cache.slot_prio), host(cache.ring)
    ck, cv = host(cache.k), host(cache.v)
    p = S - 1
    n = min(S, Bc)
    canon = orc.canonical_priority(prio)
    for b in range(nseq):
        for h in range(hkv):
            want = orc.kept_row_by_sorting(prio[b, h], p, s, w, k)
            assert len(want) == n
            assert sorted(sp[b, h, :n].tolist()) == want.tolist(), (b, h)
            assert (sp[b, h, n:] == -1).all()
            for j in range(n):
                t = int(sp[b, h, j])
                is_long = s <= t <= p - w
                want_p = np.float32(canon[b, h, t]) if is_long else np.float32(0.0)
                assert np.array_equal(np.float32(sprio[b, h, j]).view(np.uint32),
                                      want_p.view(np.uint32)), (b, h, j, t)
                assert np.array_equal(ck[b, h, j], K[b, h, t]) and np.array_equal(cv[b, h, j], V[b, h, t])
                if p - t < w:
                    assert ring[b, h, t % w] == j, (b, h, t)


def test_handoff_then_decode():
    """Decoding on from the handoff keeps the cache equal (as sets) to a cache
    decoded from position 0 and to the oracle's kept rows, and the outputs match
    the oracle's attention over them."""
    dev = device()
    nseq, hq, hkv, D, s, w, k = 2, 8, 2, 128, 3, 8, 24
    S, steps = 120, 50
    announce("handoff then decode")
    td = torch.bfloat16
    Bc = s + w + k
    T = S + steps
    prio = _rand((nseq, hkv, T), 81)
    K = _bf16(_rand((nseq, hkv, T, D), 82))
    V = _bf16(_rand((nseq, hkv, T, D), 83))
    Qd = _bf16(_rand((T, nseq, hq, D), 84))
    rank, tau = kv.thresholds(to_dev(np.ascontiguousarray(prio[:, :, :S])), s, w, k)
    ca = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    kv.cache_from_prefill(ca, to_dev(np.ascontiguousarray(K[:, :, :S]), td),
                          to_dev(np.ascontiguousarray(V[:, :, :S]), td),
                          to_dev(np.ascontiguousarray(prio[:, :, :S])), rank, tau, s, w, k)
    cb = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)

    def step(cache, p):
        u = p - w
        pl = prio[:, :, u] if u >= 0 else np.zeros((nseq, hkv), np.float32)
        return kv.decode_step(cache, to_dev(np.full(nseq, p, np.int32)), to_dev(Qd[p], td),
                              to_dev(np.ascontiguousarray(K[:, :, p]), td),
                              to_dev(np.ascontiguousarray(V[:, :, p]), td),
                              to_dev(np.ascontiguousarray(pl)), s, w, k)

    for p in range(S):
        step(cb, p)
    for p in range(S, T):
        oa, la = step(ca, p)
        step(cb, p)
        n = min(p + 1, Bc)
        spa, spb = host(ca.slot_pos)[:, :, :n], host(cb.slot_pos)[:, :, :n]
        held = []
        for b in range(nseq):
            for h in range(hkv):
                want = orc.kept_row_by_sorting(prio[b, h], p, s, w, k)
                assert sorted(spa[b, h].tolist()) == want.tolist(), (p, b, h)
                assert sorted(spb[b, h].tolist()) == want.tolist(), (p, b, h)
                held.append(want)
        for b in range(nseq):
            oo, ll = orc.decode_attention(Qd[p, b], K[b], V[b], held[b * hkv:(b + 1) * hkv])
            assert np.abs(host(oa)[b] - oo).max() <= TOL["bf16"]["o"], (p, b)
            assert np.abs(host(la)[b] - ll).max() <= TOL["bf16"]["lse"], (p, b)


# ---------------------------------------------------------------- boundary labels
LABEL_CASES = [
    # b, Hkv, S, s, w, k, n, log_gamma per head, score kind, rows (None = all)
    (1, 2, 300, 4, 16, 40, 8, (-0.3, -0.05), "normal", None),
    (2, 1, 257, 2, 5, 17, 3, (-0.5,), "ties", None),           # ties, NaN, +-inf
    (1, 2, 200, 3, 7, 0, 4, (-0.2, -0.1), "normal", None),     # k = 0
    (1, 1, 180, 1, 4, 500, 5, (-0.4,), "normal", None),        # k > S: all eligible kept
    (1, 2, 220, 0, 0, 25, 1, (-1.0, -0.01), "normal", None),   # n = 1, w = 0, s = 0
    (1, 1, 240, 2, 3, 30, 6, (0.0,), "ties", None),            # no decay
    (1, 1, 150, 2, 3, 20, 4, (-0.25,), "equal", None),         # every score equal
    (1, 1, 1500, 8, 32, 200, 16, (-0.15,), "ties", None),      # kept bin lists patched across ties
    (1, 2, 5000, 16, 64, 300, 64, (-0.1, -0.02), "normal",     # 16 keys per thread
     list(range(0, 100)) + list(range(2000, 2040)) + list(range(4900, 5000))),
    (1, 1, 20000, 16, 128, 1000, 64, (-0.05,), "ties",          # 32 keys per thread
     list(range(1100, 1160)) + list(range(19900, 20000))),
]


def _label_scores(kind, shape, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * 1.5 - 9.5).astype(np.float32)
    if kind == "ties":
        x = np.round(x * 4).astype(np.float32) / 4
        x.flat[rng.integers(0, x.size, max(1, x.size // 30))] = np.nan
        x.flat[rng.integers(0, x.size, max(1, x.size // 60))] = -np.inf
        x.flat[rng.integers(0, x.size, max(1, x.size // 60))] = np.inf
    elif kind == "equal":
        x[:] = np.float32(-3.0)
    return x


@pytest.mark.parametrize("case", LABEL_CASES,
                         ids=lambda c: "b{}h{}S{}s{}w{}k{}n{}-{}".format(*c[:7], c[8]))
def test_boundary_labels_parity(case):
    b, hkv, S, s, w, k, n, lgs, kind, rows = case
    announce(f"boundary_labels {case[:9]}")
    dev = device()
    score = _label_scores(kind, (b, hkv, S), 91)
    lg = np.array(lgs, np.float32)
    tb, y = kv.boundary_labels(to_dev(score), to_dev(lg), n, s, w, k)
    tb, y = host(tb), host(y)
    want_t, want_y = orc.boundary_labels(score, lg, n, s, w, k, rows=rows)
    sel = np.arange(S) if rows is None else np.array(rows)
    assert np.array_equal(tb[..., sel], want_t[..., sel])
    assert np.array_equal(y[..., sel], want_y[..., sel])
    if rows is not None:
        # rows the oracle skipped still carry a valid label
        assert set(np.unique(y).tolist()) <= {-1, 0, 1}
        assert ((tb >= -1) & (tb < S)).all()


# ---------------------------------------------------------------- backward
BWD_CASES = [
    # b, Hq, Hkv, S, D, s, w, k, forward output dtype
    (1, 8, 2, 300, 128, 4, 16, 40, "f32"),
    (2, 4, 1, 200, 64, 3, 9, 20, "bf16"),       # D = 64, bf16 O
    (1, 4, 4, 257, 128, 2, 7, 0, "f32"),        # k = 0, G = 1
    (1, 8, 1, 130, 128, 1, 1, 500, "f32"),      # k >= S: dense causal; w = 1; G = 8
    (1, 2, 2, 64, 128, 0, 5, 10, "f32"),        # s = 0
    (1, 8, 2, 1500, 128, 8, 64, 200, "bf16"),   # several tiles, listed long-range keys
    (1, 4, 2, 700, 64, 2, 40, 90, "f32"),       # D = 64, G = 2, split dK/dV tiles
    (1, 6, 2, 333, 128, 3, 20, 50, "bf16"),     # G = 3: odd item counts (padded items)
]


def _bwd_rounding_bounds(q, k, v, dout, rank, tau, s, w, o_bf16):
    """First-order bound on each gradient element's error from the bfloat16
    roundings of the path: the forward's probabilities in O (and O itself
    when it is bfloat16) through D_i = <dO_i, O_i>, dS before the dQ and dK
    products, P before the dV product.  Every term is taken with its largest
    rounding and its absolute value, so no cancellation can hide behind it;
    float32 sums add far less (n 2^-24 relative)."""
    b, hq, S, D = q.shape
    G = hq // k.shape[1]
    sc = orc.default_scale(D, 0.0)
    u = BF16_U
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    qs = np.arange(S)
    for bi in range(b):
        for hh in range(hq):
            h = hh // G
            K, V = k[bi, h].astype(np.float64), v[bi, h].astype(np.float64)
            Q, dO = q[bi, hh].astype(np.float64), dout[bi, hh].astype(np.float64)
            keep = orc.mask_rows(rank[bi, h], tau[bi, h, qs], qs, s, w)
            z = np.where(keep, sc * (Q @ K.T), -np.inf)
            e = np.where(keep, np.exp(z - z.max(1, keepdims=True)), 0.0)
            P = e / e.sum(1, keepdims=True)
            O = P @ V
            dS = P * (dO @ V.T - (dO * O).sum(1, keepdims=True))
            o_err = u * (P @ np.abs(V)) + (u * np.abs(O) if o_bf16 else 0.0)
            d_err = (np.abs(dO) * o_err).sum(1, keepdims=True)
            ds_err = u * np.abs(dS) + P * d_err
            bq[bi, hh] = sc * (ds_err @ np.abs(K))
            bk[bi, h] += sc * (ds_err.T @ np.abs(Q))
            bv[bi, h] += u * (P.T @ np.abs(dO))
    return bq, bk, bv


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "b{}q{}kv{}S{}D{}s{}w{}k{}-{}".format(*c))
def test_masked_attn_bwd_parity(case):
    b, hq, hkv, S, D, s, w, k, odt = case
    announce(f"masked_attn_bwd {case}")
    device()
    td = torch.bfloat16
    q = _bf16(_rand((b, hq, S, D), 101))
    kk = _bf16(_rand((b, hkv, S, D), 102, scale_keys=True))
    v = _bf16(_rand((b, hkv, S, D), 103))
    dout = _bf16(_rand((b, hq, S, D), 104))
    prio = _rand((b, hkv, S), 105)
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    o, lse = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s, w, k,
                                out_dtype=torch.float32 if odt == "f32" else td)
    dq, dk, dv = kv.masked_attn_bwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), o, lse, rank, tau,
                                    to_dev(dout, td), s, w, k)
    rank_o = orc.priority_ranks(prio)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    rq, rk, rv = orc.masked_attention_backward(q, kk, v, rank_o, tau_o, s, w, dout)
    bounds = _bwd_rounding_bounds(q, kk, v, dout, rank_o, tau_o, s, w, odt == "bf16")
    for name, got, ref, bd in zip(("dq", "dk", "dv"), (host(dq), host(dk), host(dv)),
                                  (rq, rk, rv), bounds):
        err = got.astype(np.float64) - ref
        fro = np.linalg.norm(err) / np.linalg.norm(ref)
        assert fro <= BWD_TOL[odt]["fro"], (name, fro)
        # every element within its rounding bound (plus float32 noise where
        # the bound vanishes: a row whose one kept key gives dS = 0)
        over = np.abs(err) - (bd + 1e-6 * np.abs(ref).max())
        assert (over <= 0).all(), (name, np.unravel_index(over.argmax(), over.shape), over.max())
