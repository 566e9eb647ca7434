"""GPU parity of libkvpop against the CPU oracle on reduced shapes (several tiles,
ragged tails, edge cases).  Integer outputs are compared bit-exactly; floats
within the stated tolerances.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import fixed_budget_sparse_amd as kv
import oracle as orc
from gpu_util import TOL, announce, device, host, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale_keys=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if scale_keys:
        x[..., :4, :] *= 4
    return x


def _bf16_exact(x):
    from workloads import round_to_bf16
    return round_to_bf16(x)


# ---------------------------------------------------------------- thresholds
THR_CASES = [
    # b, Hkv, S, s, w, k, prio kind
    (1, 1, 512, 4, 32, 64, "normal"),
    (1, 1, 1, 0, 1, 1, "normal"),
    (1, 2, 7, 0, 1, 0, "normal"),
    (1, 1, 100, 3, 200, 5, "normal"),        # w >= S: nothing eligible
    (2, 1, 300, 2, 5, 400, "normal"),        # k >= S: cutoff always open
    (1, 2, 5000, 16, 128, 300, "normal"),    # two sort tiles, many cutoff chunks
    (2, 3, 9000, 0, 1, 37, "ties"),          # heavy ties, NaN, +-inf
    (1, 1, 4097, 1, 1, 1, "increasing"),     # cutoff moves every step
    (1, 1, 3000, 5, 9, 100, "decreasing"),   # cutoff never moves
    (1, 2, 16384, 3, 7, 500, "ties"),        # largest one-workgroup rank
    (1, 1, 16385, 3, 7, 500, "ties"),        # smallest multi-workgroup rank
]


def _prio(kind, shape, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "ties":
        p = np.round(rng.standard_normal(shape) * 2).astype(np.float32)
        p.flat[rng.integers(0, p.size, p.size // 50)] = np.nan
        p.flat[rng.integers(0, p.size, p.size // 100)] = np.inf
        p.flat[rng.integers(0, p.size, p.size // 100)] = -np.inf
        p[p == 0] = -0.0
        return p
    S = shape[-1]
    base = np.arange(S, dtype=np.float32)
    p = np.broadcast_to(base if kind == "increasing" else -base, shape)
    return np.ascontiguousarray(p)


@pytest.mark.parametrize("case", THR_CASES, ids=lambda c: "b{}h{}S{}s{}w{}k{}-{}".format(*c))
def test_thresholds_bit_exact(case):
    b, hkv, S, s, w, k, kind = case
    announce(f"thresholds {case}")
    prio = _prio(kind, (b, hkv, S), 7)
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    torch.cuda.synchronize()
    rank_o = orc.priority_ranks(prio)
    assert np.array_equal(host(rank), rank_o)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    assert np.array_equal(host(tau), tau_o)
    if S <= 600:
        _, tau_s = orc.thresholds_by_sorting(prio, s, w, k)
        assert np.array_equal(host(tau), tau_s)


def test_thresholds_deterministic():
    device()
    prio = _prio("ties", (1, 2, 6000), 3)
    r1, t1 = kv.thresholds(to_dev(prio), 3, 17, 200)
    r2, t2 = kv.thresholds(to_dev(prio), 3, 17, 200)
    assert torch.equal(r1, r2) and torch.equal(t1, t2)


# ---------------------------------------------------------------- forward
FWD_CASES = [
    # b, Hq, Hkv, S, D, s, w, k, dtype
    (1, 2, 1, 512, 64, 4, 32, 64, "f32"),       # the tiny float32 workload
    (1, 8, 2, 777, 128, 4, 40, 100, "bf16"),    # G=4, ragged tail
    (2, 4, 2, 300, 64, 3, 17, 50, "bf16"),      # G=2, D=64, batch 2
    (1, 3, 3, 400, 128, 2, 9, 31, "bf16"),      # G=1 (128 rows per head)
    (1, 16, 2, 350, 128, 0, 1, 20, "bf16"),     # G=8, s=0, w=1
    (1, 4, 1, 260, 128, 5, 11, 1000, "bf16"),   # k >= S: dense causal
    (1, 4, 1, 260, 128, 5, 11, 0, "bf16"),      # k = 0: sinks + window
    (1, 4, 2, 5, 128, 1, 2, 1, "bf16"),         # S smaller than a tile
    (1, 6, 2, 333, 128, 4, 20, 64, "bf16"),     # G=3 (rows padded)
]


def _fwd_inputs(b, hq, hkv, S, D, dtype, seed):
    q = _rand((b, hq, S, D), seed)
    k = _rand((b, hkv, S, D), seed + 1, scale_keys=True)
    v = _rand((b, hkv, S, D), seed + 2)
    if dtype == "bf16":
        q, k, v = (_bf16_exact(x) for x in (q, k, v))
    prio = _rand((b, hkv, S), seed + 3)
    return q, k, v, prio


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "b{}q{}kv{}S{}D{}s{}w{}k{}-{}".format(*c))
def test_masked_fwd_parity(case):
    b, hq, hkv, S, D, s, w, k, dt = case
    announce(f"masked_fwd {case}")
    q, kk, v, prio = _fwd_inputs(b, hq, hkv, S, D, dt, 11)
    td = tdtype(dt)
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    o, lse = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s, w, k,
                                out_dtype=torch.float32)
    o_bf, lse_bf = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s,
                                      w, k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rank_o = orc.priority_ranks(prio)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    O, LSE = orc.masked_attention(q, kk, v, rank_o, tau_o, s, w)
    tol = TOL[dt]
    og, lg = host(o), host(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert np.abs(og - O).max() <= tol["o"], np.abs(og - O).max()
    assert np.abs(lg - LSE).max() <= tol["lse"], np.abs(lg - LSE).max()
    # bfloat16 output = the float32 output rounded, within one bf16 ulp
    ob = host(o_bf)
    ulp = np.maximum(np.abs(og), 1e-30)
    ulp = 2.0 ** (np.floor(np.log2(ulp)) - 7)
    assert (np.abs(ob - og) <= ulp + 1e-30).all()
    assert torch.equal(lse_bf, lse)


def test_masked_fwd_far_logit_reruns_exact():
    """The forward takes each row's maximum over its first key chunk as the
    reference for the whole tile and checks the row sums at the end; a kept
    key whose logit lies about 800 above that reference (far beyond float32's
    exponent range) makes the tile run again with a running maximum.  Both
    bf16 and float32 outputs match the oracle (float64)."""
    device()
    b, hq, hkv, S, D, s, w, k = 1, 8, 2, 700, 128, 4, 40, 100
    announce("masked_fwd far logit: exact rerun")
    q, kk, v, prio = _fwd_inputs(b, hq, hkv, S, D, "bf16", 19)
    t_star, row = 500, 520                      # in the window of rows 500..539
    u = q[0, 0, row].astype(np.float64)
    kk[0, 0, t_star] = (u * (800.0 * np.sqrt(D) / (u @ u))).astype(np.float32)
    kk = _bf16_exact(kk)
    td = torch.bfloat16
    rank, tau = kv.thresholds(to_dev(prio), s, w, k)
    outs = [kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, s, w, k,
                               out_dtype=dt) for dt in (torch.float32, torch.bfloat16)]
    torch.cuda.synchronize()
    rank_o = orc.priority_ranks(prio)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    O, LSE = orc.masked_attention(q, kk, v, rank_o, tau_o, s, w)
    assert LSE[0, 0, row] > 700
    for o, lse in outs:
        og, lg = host(o), host(lse)
        assert np.isfinite(og).all() and np.isfinite(lg).all()
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(O), 1e-30))) - 8)
        assert (np.abs(og - O) - ulp).max() <= TOL["bf16"]["o"]
        assert np.abs(lg - LSE).max() <= TOL["bf16"]["lse"], np.abs(lg - LSE).max()


# ---------------------------------------------------------------- target
TGT_CASES = [
    (1, 2, 1, 512, 64, 32, "f32"),
    (1, 8, 2, 700, 128, 33, "bf16"),
    (2, 4, 2, 300, 64, 0, "bf16"),        # w = 0
    (1, 4, 4, 257, 128, 1, "bf16"),       # G = 1, ragged
    (1, 4, 1, 200, 128, 300, "bf16"),     # w >= S: all -inf
]


@pytest.mark.parametrize("case", TGT_CASES, ids=lambda c: "b{}q{}kv{}S{}D{}w{}-{}".format(*c))
def test_future_target_parity(case):
    b, hq, hkv, S, D, w, dt = case
    announce(f"future_target {case}")
    q, kk, _, _ = _fwd_inputs(b, hq, hkv, S, D, dt, 21)
    td = tdtype(dt)
    _, LSE = orc.dense_causal_attention(q, kk, kk)          # teacher LSE from the oracle
    tgt = kv.future_target(to_dev(q, td), to_dev(kk, td), to_dev(LSE.astype(np.float32)), w)
    torch.cuda.synchronize()
    T = orc.future_target_colsum(q, kk, LSE.astype(np.float32).astype(np.float64), w)
    tg = host(tgt)
    assert np.array_equal(np.isneginf(tg), np.isneginf(T))
    sel = T > -20
    if sel.any():
        err = np.abs(tg[sel] - T[sel]).max()
        assert err <= TOL[dt]["tgt"], err
    if w == 0:
        assert np.abs(np.exp(tg.astype(np.float64)).sum(-1) - S).max() < 2e-3 * S


def test_target_with_gpu_dense_lse_matches_w0_total():
    """k >= S makes the forward dense causal; its LSE drives the target, and with
    w = 0 the column masses of every head sum to S."""
    device()
    b, hq, hkv, S, D = 1, 8, 2, 640, 128
    q, kk, v, prio = _fwd_inputs(b, hq, hkv, S, D, "bf16", 31)
    td = torch.bfloat16
    rank, tau = kv.thresholds(to_dev(prio), 0, 1, S)
    _, lse = kv.masked_attn_fwd(to_dev(q, td), to_dev(kk, td), to_dev(v, td), rank, tau, 0, 1, S)
    tgt = kv.future_target(to_dev(q, td), to_dev(kk, td), lse, 0)
    tot = torch.exp(tgt.double()).sum(-1)
    assert (tot - S).abs().max().item() < 1e-3 * S


# ---------------------------------------------------------------- decode
DEC_CASES = [
    # nseq, Hq, Hkv, D, s, w, k, steps, dtype
    (3, 8, 2, 128, 2, 8, 12, 90, "bf16"),
    (2, 4, 2, 64, 0, 3, 5, 60, "f32"),
    (2, 4, 1, 128, 4, 5, 0, 40, "bf16"),       # k = 0
    (1, 2, 1, 128, 1, 2, 300, 200, "bf16"),    # budget larger than the run: 3 splits, partial fill
    (2, 8, 2, 64, 3, 20, 400, 640, "f32"),     # 4 splits past the fill, D = 64, float32
    (1, 4, 1, 128, 4, 300, 0, 420, "bf16"),    # 3 splits past the fill, k = 0
    (1, 2, 1, 64, 2, 30, 1568, 1700, "bf16"),  # one pair, B = 1600: 13 splits (the 16-split merge)
    (1, 2, 1, 64, 2, 30, 2268, 2400, "bf16"),  # one pair, B = 2300: 18 splits (the looping merge)
]


def _slot_sets(cache, p, Bc):
    sp = host(cache.slot_pos)
    n = min(p + 1, Bc)
    return [[sorted(sp[b, h, :n].tolist()) for h in range(sp.shape[1])] for b in range(sp.shape[0])]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "n{}q{}kv{}D{}s{}w{}k{}T{}-{}".format(*c))
def test_decode_parity(case):
    nseq, hq, hkv, D, s, w, k, steps, dt = case
    announce(f"decode {case}")
    dev = device()
    td = tdtype(dt)
    Bc = s + w + k
    rng = np.random.default_rng(41)
    prio_table = rng.standard_normal((nseq, hkv, steps)).astype(np.float32)
    Ks = rng.standard_normal((nseq, hkv, steps, D)).astype(np.float32)
    Vs = rng.standard_normal((nseq, hkv, steps, D)).astype(np.float32)
    Qs = rng.standard_normal((steps, nseq, hq, D)).astype(np.float32)
    if dt == "bf16":
        Ks, Vs, Qs = (_bf16_exact(x) for x in (Ks, Vs, Qs))
    cache = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    states = [[orc.DecodeState(s, w, k) for _ in range(hkv)] for _ in range(nseq)]
    tol = TOL[dt]
    for p in range(steps):
        u = p - w
        pl = prio_table[:, :, u] if u >= 0 else np.zeros((nseq, hkv), np.float32)
        o, lse = kv.decode_step(cache, to_dev(np.full(nseq, p, np.int32)), to_dev(Qs[p], td),
                                to_dev(np.ascontiguousarray(Ks[:, :, p]), td),
                                to_dev(np.ascontiguousarray(Vs[:, :, p]), td), to_dev(pl),
                                s, w, k)
        for bi in range(nseq):
            for h in range(hkv):
                states[bi][h].step(p, float(prio_table[bi, h, u]) if u >= s else float("nan"))
        got = _slot_sets(cache, p, Bc)
        for bi in range(nseq):
            held = [states[bi][h].held() for h in range(hkv)]
            for h in range(hkv):
                assert got[bi][h] == held[h].tolist(), (p, bi, h)
            oo, ll = orc.decode_attention(Qs[p, bi], Ks[bi], Vs[bi], held)
            assert np.abs(host(o)[bi] - oo).max() <= tol["o"], (p, bi)
            assert np.abs(host(lse)[bi] - ll).max() <= tol["lse"], (p, bi)


def test_decode_reset_and_skip():
    """A sequence restarting at p = 0 in the middle of a batch, and a skipped
    sequence (p < 0) whose cache stays untouched."""
    dev = device()
    nseq, hq, hkv, D, s, w, k = 3, 4, 1, 128, 1, 4, 6
    Bc = s + w + k
    rng = np.random.default_rng(5)
    cache = kv.new_decode_cache(nseq, hkv, D, s, w, k, device=dev)
    states = [orc.DecodeState(s, w, k) for _ in range(nseq)]
    toks = {b: [] for b in range(nseq)}
    pos = [0, 0, 0]
    for step in range(40):
        if step == 20:
            pos[1] = 0
            states[1] = orc.DecodeState(s, w, k)
            toks[1] = []
        skip = step % 7 == 3
        q = _bf16_exact(rng.standard_normal((nseq, hq, D)).astype(np.float32))
        kn = _bf16_exact(rng.standard_normal((nseq, hkv, D)).astype(np.float32))
        vn = _bf16_exact(rng.standard_normal((nseq, hkv, D)).astype(np.float32))
        pl = rng.standard_normal((nseq, hkv)).astype(np.float32)
        pvec = np.array(pos, np.int32)
        if skip:
            pvec[2] = -1
        before = cache.clone()
        o, lse = kv.decode_step(cache, to_dev(pvec), to_dev(q, torch.bfloat16),
                                to_dev(kn, torch.bfloat16), to_dev(vn, torch.bfloat16),
                                to_dev(pl), s, w, k)
        for b in range(nseq):
            if pvec[b] < 0:
                assert torch.equal(cache.slot_pos[b], before.slot_pos[b])
                assert torch.equal(cache.k[b], before.k[b])
                assert (host(o)[b] == 0).all() and np.isneginf(host(lse)[b]).all()
                continue
            p = int(pvec[b])
            toks[b].append((kn[b, 0], vn[b, 0]))
            # the priority passed at step p is that of token p - w
            states[b].step(p, float(pl[b, 0]) if p - w >= s else float("nan"))
            pos[b] += 1
            held = states[b].held()
            n = min(p + 1, Bc)
            assert sorted(host(cache.slot_pos)[b, 0, :n].tolist()) == held.tolist(), (step, b)
            kk = np.stack([toks[b][t][0] for t in range(p + 1)])[None]
            vv = np.stack([toks[b][t][1] for t in range(p + 1)])[None]
            oo, ll = orc.decode_attention(q[b], kk, vv, [held])
            assert np.abs(host(o)[b] - oo).max() <= 1e-2
            assert np.abs(host(lse)[b] - ll).max() <= 1e-3
    # membership check at the end against the explicit simulation
    sp = host(cache.slot_pos)
    for b in range(nseq):
        n = min(pos[b], Bc)
        assert sorted(sp[b, 0, :n].tolist()) == states[b].held().tolist(), b
