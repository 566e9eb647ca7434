"""GPU parity on the edge cases of the exact rows: decode and the prefill ->
decode handoff under tied, NaN, +-inf and signed-zero priorities, and the tiny
float32 workload drawn exactly as its recipe states (seed 0).

The decode rules these cases exercise ([Notes] §2.2: the newcomer t_new = q - w
enters E(q); §2.3: tokens are ranked by their static priority): the token
leaving the window replaces the worst held long-range token only when its
priority is strictly larger, the worst among equal priorities is the one with
the highest position, NaN counts as -inf and -0 as +0.  Cache membership is
compared with the oracle's explicit decode simulation bit for bit at every
step, outputs within the bf16 tolerances."""
import numpy as np
import pytest
import torch

import fixed_budget_sparse_amd as kv
import oracle as orc
import workloads as W
from gpu_util import TOL, announce, device, host, tdtype, to_dev

pytestmark = pytest.mark.gpu

# priorities drawn from a small set so that ties are the rule, not the exception
TIE_VALUES = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], np.float32)


def _tie_table(shape, seed):
    rng = np.random.default_rng(seed)
    return TIE_VALUES[rng.integers(0, len(TIE_VALUES), shape)].astype(np.float32)


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


DEC_TIE_CASES = [
    # nseq, Hq, Hkv, D, s, w, k, steps, dtype
    (3, 8, 2, 128, 2, 4, 6, 160, "bf16"),      # one workgroup per (sequence, head)
    (2, 4, 2, 64, 0, 3, 5, 100, "f32"),        # s = 0, float32 cache
    (1, 4, 1, 128, 1, 2, 300, 420, "bf16"),    # split cache: 300 long-range slots, mostly tied
    (2, 8, 2, 128, 3, 5, 1, 80, "bf16"),       # k = 1: every leaving token meets the one held
]


@pytest.mark.parametrize("case", DEC_TIE_CASES,
                         ids=lambda c: "n{}q{}kv{}D{}s{}w{}k{}T{}-{}".format(*c))
def test_decode_ties_bit_exact(case):
    nseq, hq, hkv, D, s, w, k, steps, dt = case
    announce(f"decode ties {case}")
    dev = device()
    td = tdtype(dt)
    Bc = s + w + k
    rng = np.random.default_rng(131)
    prio_table = _tie_table((nseq, hkv, steps), 132)
    Ks = rng.standard_normal((nseq, hkv, steps, D)).astype(np.float32)
    Vs = rng.standard_normal((nseq, hkv, steps, D)).astype(np.float32)
    Qs = rng.standard_normal((steps, nseq, hq, D)).astype(np.float32)
    if dt == "bf16":
        Ks, Vs, Qs = (W.round_to_bf16(x) for x in (Ks, Vs, Qs))
    canon = orc.canonical_priority(prio_table)
    cache = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    # the same steps on a cache without the next-step record (every full step
    # scans its slots): outputs and arrays must agree bit for bit
    bare = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    bare.state = None
    stale_at = {Bc + 3, steps - 7}   # steps entered with the record marked stale
    states = [[orc.DecodeState(s, w, k) for _ in range(hkv)] for _ in range(nseq)]
    tol = TOL[dt]
    n_equal_worst = 0   # leaving token equal to the worst held one (it must stay out)
    for p in range(steps):
        u = p - w
        pl = prio_table[:, :, u] if u >= 0 else np.zeros((nseq, hkv), np.float32)
        for bi in range(nseq):
            for h in range(hkv):
                st = states[bi][h]
                if u >= s and len(st.long) == k and k > 0:
                    worst = min(st.long.values())
                    n_equal_worst += int(canon[bi, h, u] == worst)
        if p in stale_at:
            cache.state[..., 0] = 0
        args = (to_dev(np.full(nseq, p, np.int32)), to_dev(Qs[p], td),
                to_dev(np.ascontiguousarray(Ks[:, :, p]), td),
                to_dev(np.ascontiguousarray(Vs[:, :, p]), td), to_dev(pl), s, w, k)
        o, lse = kv.decode_step(cache, *args)
        o2, lse2 = kv.decode_step(bare, *args)
        assert torch.equal(o.view(torch.int32), o2.view(torch.int32)), p
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), p
        for x, y in zip(cache.arrays()[:5], bare.arrays()):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), p
        for bi in range(nseq):
            for h in range(hkv):
                states[bi][h].step(p, float(prio_table[bi, h, u]) if u >= s else float("nan"))
        # the record for step p + 1: the worst held long-range token (lowest
        # priority, ties to the highest position), or none
        rec = host(cache.state)
        for bi in range(nseq):
            for h in range(hkv):
                lr = states[bi][h].long
                r = rec[bi, h]
                assert r[0] == p + 1, (p, bi, h)
                if not lr:
                    assert r[3] == -1, (p, bi, h)
                    continue
                t = min(lr, key=lambda x: (lr[x], -x))
                assert r[2] == t and r[1] == _bits(canon[bi, h, t]).view(np.int32), (p, bi, h)
                assert host(cache.slot_pos)[bi, h, r[3]] == t, (p, bi, h)
        n = min(p + 1, Bc)
        sp, spr = host(cache.slot_pos), host(cache.slot_prio)
        oh, lh = host(o), host(lse)
        for bi in range(nseq):
            held = [states[bi][h].held() for h in range(hkv)]
            for h in range(hkv):
                assert sorted(sp[bi, h, :n].tolist()) == held[h].tolist(), (p, bi, h)
                # long-range slots carry the canonical priority (NaN -> -inf, -0 -> +0)
                for j in range(n):
                    t = int(sp[bi, h, j])
                    if s <= t <= p - w:
                        assert _bits(spr[bi, h, j]) == _bits(canon[bi, h, t]), (p, bi, h, t)
            oo, ll = orc.decode_attention(Qs[p, bi], Ks[bi], Vs[bi], held)
            assert np.abs(oh[bi] - oo).max() <= tol["o"], (p, bi)
            assert np.abs(lh[bi] - ll).max() <= tol["lse"], (p, bi)
    # the strict-'>' case actually occurred (equal priorities, leaving token dropped)
    if k > 0:
        assert n_equal_worst > 0


def test_handoff_then_decode_ties():
    """A prompt with tied, NaN and +-inf priorities handed over to the cache,
    then decoded on with tied priorities: membership equals the oracle's
    explicit decode from position 0 at every step."""
    dev = device()
    nseq, hq, hkv, D, s, w, k = 2, 8, 2, 128, 3, 6, 20
    S, steps = 150, 90
    announce("handoff then decode, tied priorities")
    td = torch.bfloat16
    Bc = s + w + k
    T = S + steps
    prio = _tie_table((nseq, hkv, T), 141)
    rng = np.random.default_rng(142)
    K = W.round_to_bf16(rng.standard_normal((nseq, hkv, T, D)).astype(np.float32))
    V = W.round_to_bf16(rng.standard_normal((nseq, hkv, T, D)).astype(np.float32))
    Qd = W.round_to_bf16(rng.standard_normal((T, nseq, hq, D)).astype(np.float32))
    pp = np.ascontiguousarray(prio[:, :, :S])
    rank, tau = kv.thresholds(to_dev(pp), s, w, k)
    cache = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=td, device=dev)
    kv.cache_from_prefill(cache, to_dev(np.ascontiguousarray(K[:, :, :S]), td),
                          to_dev(np.ascontiguousarray(V[:, :, :S]), td), to_dev(pp), rank, tau,
                          s, w, k)
    states = [[orc.DecodeState(s, w, k) for _ in range(hkv)] for _ in range(nseq)]
    for p in range(S):
        u = p - w
        for bi in range(nseq):
            for h in range(hkv):
                states[bi][h].step(p, float(prio[bi, h, u]) if u >= s else float("nan"))
    torch.cuda.synchronize()
    n = min(S, Bc)
    sp = host(cache.slot_pos)
    for bi in range(nseq):
        for h in range(hkv):
            assert sorted(sp[bi, h, :n].tolist()) == states[bi][h].held().tolist(), (bi, h)
    # the handoff marks the next-step record stale: the first step scans the
    # slots, and every step leaves the record of the worst long-range token
    assert (host(cache.state)[..., 0] == 0).all()
    canon = orc.canonical_priority(prio)
    for p in range(S, T):
        u = p - w
        o, lse = kv.decode_step(cache, to_dev(np.full(nseq, p, np.int32)), to_dev(Qd[p], td),
                                to_dev(np.ascontiguousarray(K[:, :, p]), td),
                                to_dev(np.ascontiguousarray(V[:, :, p]), td),
                                to_dev(np.ascontiguousarray(prio[:, :, u])), s, w, k)
        for bi in range(nseq):
            for h in range(hkv):
                states[bi][h].step(p, float(prio[bi, h, u]) if u >= s else float("nan"))
        n = min(p + 1, Bc)
        sp = host(cache.slot_pos)
        for bi in range(nseq):
            held = [states[bi][h].held() for h in range(hkv)]
            for h in range(hkv):
                assert sorted(sp[bi, h, :n].tolist()) == held[h].tolist(), (p, bi, h)
                # the same set as the forward's kept row p (static priorities)
                assert np.array_equal(held[h], orc.kept_row_by_sorting(prio[bi, h], p, s, w, k))
            oo, ll = orc.decode_attention(Qd[p, bi], K[bi], V[bi], held)
            assert np.abs(host(o)[bi] - oo).max() <= TOL["bf16"]["o"], (p, bi)
            assert np.abs(host(lse)[bi] - ll).max() <= TOL["bf16"]["lse"], (p, bi)
        rec = host(cache.state)
        for bi in range(nseq):
            for h in range(hkv):
                lr = states[bi][h].long
                t = min(lr, key=lambda x: (lr[x], -x))
                assert rec[bi, h, 0] == p + 1 and rec[bi, h, 2] == t, (p, bi, h)
                assert rec[bi, h, 1] == _bits(canon[bi, h, t]).view(np.int32), (p, bi, h)


def test_tiny_workload_seed0():
    """The tiny float32 workload exactly as drawn by its recipe (S = 512, D = 64,
    G = 2, s 4, w 32, k 64, seed 0): ranks, cutoffs and kept sets bit-exact,
    the float32 forward, the dense teacher LSE and the future target against
    the oracle on every row."""
    wl = W.TINY
    announce("tiny f32 workload, seed 0")
    device()
    x = W.make_prefill(wl)
    s, w, k, S = wl.sink, wl.window, wl.topk, wl.seq_len
    td = torch.float32
    q, kk, v = (to_dev(x[n], td) for n in ("q", "k", "v"))
    rank, tau = kv.thresholds(to_dev(x["prio"]), s, w, k)
    o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=torch.float32)
    rank_d, tau_d = kv.thresholds(to_dev(x["prio"]), s, w, S)
    _, lse_dense = kv.masked_attn_fwd(q, kk, v, rank_d, tau_d, s, w, S, out_dtype=torch.float32)
    tgt = kv.future_target(q, kk, lse_dense, w)
    torch.cuda.synchronize()
    rank_o, tau_o = orc.thresholds_by_sorting(x["prio"], s, w, k)
    assert np.array_equal(host(rank), rank_o)
    assert np.array_equal(host(tau), tau_o)
    # the kept rows derived from (rank, tau) equal the sorted kept sets
    for q_ in (0, s + w - 1, s + w, s + w + k, S - 1):
        m = orc.mask_rows(host(rank)[0, 0], host(tau)[0, 0, [q_]], np.array([q_]), s, w)[0]
        assert np.array_equal(np.flatnonzero(m), orc.kept_row_by_sorting(x["prio"][0, 0], q_,
                                                                         s, w, k))
    O, L = orc.masked_attention(x["q"], x["k"], x["v"], rank_o, tau_o, s, w)
    tol = TOL["f32"]
    assert np.abs(host(o) - O).max() <= tol["o"], np.abs(host(o) - O).max()
    assert np.abs(host(lse) - L).max() <= tol["lse"], np.abs(host(lse) - L).max()
    _, LD = orc.dense_causal_attention(x["q"], x["k"], x["v"])
    assert np.abs(host(lse_dense) - LD).max() <= tol["lse"]
    T = orc.future_target_colsum(x["q"], x["k"], host(lse_dense).astype(np.float64), w)
    tg = host(tgt)
    assert np.array_equal(np.isneginf(tg), np.isneginf(T))
    sel = T > -20
    assert np.abs(tg[sel] - T[sel]).max() <= tol["tgt"], np.abs(tg[sel] - T[sel]).max()


def test_reversed_launch_order_bit_identical():
    """Every tile of the forward, the target and the backward is computed by
    one workgroup from its own inputs, so the order in which workgroups run
    must not change a bit of any output: the same calls with the launch
    order reversed (last tile first) are compared bit for bit.  S = 4096
    gives 64 forward tiles per KV head and dK/dV tiles that are split in two."""
    dev = device()
    announce("reversed launch order")
    b, hq, hkv, S, D = 1, 8, 2, 4096, 128
    s, w, k = 8, 256, 700
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    bf = torch.bfloat16
    q = torch.randn((b, hq, S, D), generator=g, device=dev).to(bf)
    kk = torch.randn((b, hkv, S, D), generator=g, device=dev).to(bf)
    v = torch.randn((b, hkv, S, D), generator=g, device=dev).to(bf)
    prio = torch.randn((b, hkv, S), generator=g, device=dev)
    dout = torch.randn((b, hq, S, D), generator=g, device=dev).to(bf)

    def run():
        rank, tau = kv.thresholds(prio, s, w, k)
        o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf)
        rank_d, tau_d = kv.thresholds(prio, 0, 1, S)                   # k >= S: dense causal
        _, lse_d = kv.masked_attn_fwd(q, kk, v, rank_d, tau_d, 0, 1, S)
        tgt = kv.future_target(q, kk, lse_d, w)
        dq, dk, dv = kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k)
        torch.cuda.synchronize()
        return [x.clone() for x in (o, lse, lse_d, tgt, dq, dk, dv)]

    ref = run()
    try:
        kv.debug_reverse_launch_order(True)
        rev = run()
    finally:
        kv.debug_reverse_launch_order(False)
    names = ("o", "lse", "dense lse", "target", "dq", "dk", "dv")
    for n, a, c in zip(names, ref, rev):
        assert torch.equal(a.view(torch.int16 if a.dtype == bf else torch.int32),
                           c.view(torch.int16 if c.dtype == bf else torch.int32)), n
