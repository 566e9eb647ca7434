"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times: the Qwen3-4B-shaped layer (S = 16384, B = 2048), the
Qwen3-8B-shaped layer (S = 32768, B = 4096), the long-context layer
(S = 131072, B = 4096), the 64-sequence decode at B = 2048 and the 8-sequence
decode over 131072 steps.

The oracle cannot evaluate these sizes whole, so outputs are compared where it
can compute them one by one: every rank, the cutoffs of every row (or of a
sample of rows plus all boundary rows at S = 131072), the forward on sampled
query rows of every head and on every row of the four query heads of one KV
head, the teacher LSE of every row and the future target on every token of
those four heads (sampled tokens at S = 32768) with the teacher LSE computed
by the oracle, and decode cache membership of every (sequence, KV head) plus
outputs of a few sequences at sampled steps.  The every-row checks run the
oracle in worker processes (``oracle_pool``).  Inputs are drawn on the device by the seeded
generators of ``workloads``; host copies feed the oracle."""
import numpy as np
import pytest
import torch

import fixed_budget_sparse_amd as kv
import oracle as orc
import workloads as W
import oracle_pool
from gpu_util import BWD_TOL, TOL, announce, device, host

pytestmark = pytest.mark.gpu

PREFILL = {"qwen3-4b-S16384": W.QWEN3_4B_S16K, "qwen3-8b-S32768": W.QWEN3_8B_S32K,
           "long-S131072": W.LONG_S128K}


def _boundary_rows(S, s, w, B, extra, seed):
    """Rows at every boundary the mask and the tiling have, plus random rows."""
    base = [0, 1, 2, 3, s - 1, s, s + 1, w - 2, w - 1, w, w + 1, s + w - 1, s + w, s + w + 1,
            B - 1, B, B + 1, B + w - 1, B + w, 63, 64, 127, 128, 255, 256, 511, 512,
            S // 2, S - 257, S - 256, S - 65, S - 64, S - 2, S - 1]
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.array(base), rng.integers(0, S, extra)])
    return np.unique(rows[(rows >= 0) & (rows < S)])


def _bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x|: the rounding of a bfloat16 output itself,
    allowed on top of the computation's tolerance."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def _inputs(wl):
    dev = device()
    x = W.make_prefill_device(wl, dev)
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name", list(PREFILL))
def test_full_thresholds(name):
    wl = PREFILL[name]
    announce(f"full thresholds {name}")
    dev = device()
    S, s, w, k = wl.seq_len, wl.sink, wl.window, wl.topk
    prio_d = W.make_prefill_device(wl, dev)["prio"]
    rank, tau = kv.thresholds(prio_d, s, w, k)
    torch.cuda.synchronize()
    prio = host(prio_d)
    rank_o = orc.priority_ranks(prio)
    assert np.array_equal(host(rank), rank_o)
    if S <= 32768:
        rows = np.arange(S)
    else:
        rows = np.union1d(_boundary_rows(S, s, w, s + w + k, 256, 3), np.arange(0, S, 509))
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k, rows=rows)
    assert np.array_equal(host(tau)[..., rows], tau_o)


@pytest.mark.parametrize("name", list(PREFILL))
def test_full_masked_fwd_sampled_rows(name):
    wl = PREFILL[name]
    announce(f"full masked_fwd {name}")
    S, s, w, k = wl.seq_len, wl.sink, wl.window, wl.topk
    x = _inputs(wl)
    rank, tau = kv.thresholds(x["prio"], s, w, k)
    o, lse = kv.masked_attn_fwd(x["q"], x["k"], x["v"], rank, tau, s, w, k,
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _boundary_rows(S, s, w, s + w + k, 48 if S > 32768 else 96, 5)
    rank_o = orc.priority_ranks(host(x["prio"]))
    tau_full = np.zeros(rank_o.shape, np.int64)
    tau_full[..., rows] = orc.thresholds_by_selection(rank_o, s, w, k, rows=rows)
    q_rows = host(x["q"][:, :, torch.as_tensor(rows, device=x["q"].device)])
    # masked_attention indexes q by row number: place the sampled rows in a
    # zero array of the full shape only along the sampled rows' positions
    qh = np.zeros(x["q"].shape, np.float32)
    qh[:, :, rows] = q_rows
    O, LSE = orc.masked_attention(qh, host(x["k"]), host(x["v"]), rank_o, tau_full, s, w,
                                  rows=rows)
    og = host(o)[:, :, rows]
    lg = host(lse)[:, :, rows]
    tol = TOL["bf16"]
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    err = np.abs(og - O) - _bf16_half_ulp(np.maximum(np.abs(O), np.abs(og)))
    assert err.max() <= tol["o"], err.max()
    assert np.abs(lg - LSE).max() <= tol["lse"], np.abs(lg - LSE).max()


# one KV head checked on every row: KV head 1 at S = 16384, the last KV head
# at S = 32768 (its four query heads)
EVERY_ROW_HEAD = {"qwen3-4b-S16384": 1, "qwen3-8b-S32768": 7}


@pytest.mark.parametrize("name", ["qwen3-4b-S16384", "qwen3-8b-S32768"])
def test_full_masked_fwd_one_kv_head_every_row(name):
    """The forward of the whole layer, in the benchmark's launch configuration
    (bf16 output); the oracle evaluates every row of the four query heads of
    one KV head, so every tile, the long-range key lists of every tile and
    the ragged end are checked."""
    wl = PREFILL[name]
    h = EVERY_ROW_HEAD[name]
    G = wl.group
    announce(f"full masked_fwd {name}, every row of KV head {h}")
    S, s, w, k = wl.seq_len, wl.sink, wl.window, wl.topk
    x = _inputs(wl)
    rank, tau = kv.thresholds(x["prio"], s, w, k)
    o, lse = kv.masked_attn_fwd(x["q"], x["k"], x["v"], rank, tau, s, w, k,
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    qs = slice(h * G, (h + 1) * G)
    rank_o = orc.priority_ranks(host(x["prio"][:, h:h + 1]))
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    assert np.array_equal(host(tau[:, h:h + 1]), tau_o)
    O, LSE = oracle_pool.masked_attention_all_rows(host(x["q"][:, qs]), host(x["k"][:, h:h + 1]),
                                                   host(x["v"][:, h:h + 1]), rank_o, tau_o, s, w)
    og, lg = host(o[:, qs]), host(lse[:, qs])
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    err = np.abs(og - O) - _bf16_half_ulp(np.maximum(np.abs(O), np.abs(og)))
    assert err.max() <= TOL["bf16"]["o"], err.max()
    assert np.abs(lg - LSE).max() <= TOL["bf16"]["lse"], np.abs(lg - LSE).max()


@pytest.mark.parametrize("name", ["qwen3-4b-S16384", "qwen3-8b-S32768"])
def test_full_teacher_lse_and_target(name):
    """The dense teacher (k >= S) and the future target of the whole layer;
    the oracle evaluates the teacher LSE of every row and the target of every
    token (of sampled tokens at S = 32768) of the four query heads of one KV
    head, with the target driven by the oracle's teacher LSE (the other heads
    receive the GPU's teacher LSE)."""
    wl = PREFILL[name]
    h = EVERY_ROW_HEAD[name]
    G = wl.group
    qs = slice(h * G, (h + 1) * G)
    announce(f"full target {name}, KV head {h}")
    S, s, w = wl.seq_len, wl.sink, wl.window
    x = _inputs(wl)
    rank_d, tau_d = kv.thresholds(x["prio"], s, w, S)
    _, lse_dense = kv.masked_attn_fwd(x["q"], x["k"], x["v"], rank_d, tau_d, s, w, S,
                                      out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    qh = host(x["q"][:, qs])
    kh = host(x["k"][:, h:h + 1])
    L = oracle_pool.dense_lse_all_rows(qh, kh)                  # teacher LSE [1, G, S]
    assert np.abs(host(lse_dense[:, qs]) - L).max() <= TOL["bf16"]["lse"]
    L32 = L.astype(np.float32)
    lse_in = lse_dense.clone()
    lse_in[:, qs] = torch.from_numpy(L32).to(lse_in.device)
    tgt = kv.future_target(x["q"], x["k"], lse_in, w)
    torch.cuda.synchronize()
    ts = np.arange(S) if S <= 16384 else _boundary_rows(S, s, w, 2048, 1024, 9)
    T = oracle_pool.future_target_all_tokens(qh, kh, L32.astype(np.float64), w, ts=ts)
    tg = host(tgt[:, qs])[..., ts]
    assert np.array_equal(np.isneginf(tg), np.isneginf(T))
    sel = T > -20
    assert sel.sum() > T.size // 2
    assert np.abs(tg[sel] - T[sel]).max() <= TOL["bf16"]["tgt"], np.abs(tg[sel] - T[sel]).max()


def _held_sets(cache, rank_o, p, s, w, k, Bc):
    """Cache membership of every (sequence, KV head) after row p, checked
    against the oracle's kept set of that row; returns the sets."""
    nseq, Hkv = rank_o.shape[:2]
    n = min(p + 1, Bc)
    sp = host(cache.slot_pos)
    assert (sp[:, :, n:] == -1).all(), p
    sp = sp[:, :, :n]
    tau = orc.thresholds_by_selection(rank_o, s, w, k, rows=[p])[..., 0]   # [nseq, Hkv]
    held = {}
    for b in range(nseq):
        for h in range(Hkv):
            keep = orc.mask_rows(rank_o[b, h, :p + 1], tau[b, h:h + 1], np.array([p]), s, w)[0]
            want = np.flatnonzero(keep)
            assert len(want) == n, (p, b, h)
            assert np.array_equal(np.sort(sp[b, h]), want), (p, b, h)
            held[(b, h)] = want
    return held


def _decode_run(wl, n_steps, check_steps, out_seqs, handoff_at=0):
    """Runs decode steps over every sequence; at each step of ``check_steps``
    compares cache membership of every (sequence, KV head) with the oracle's
    kept set of that row, and o/LSE of ``out_seqs``.  With ``handoff_at`` > 0
    the cache is first filled from a prompt of that many tokens
    (kvpop_thresholds + kvpop_cache_from_prefill, checked the same way, with
    its K/V rows and long-range priorities) and decoding starts there."""
    dev = device()
    nseq, Hq, Hkv, D = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    s, w, k = wl.sink, wl.window, wl.topk
    Bc = s + w + k
    st = W.make_decode_stream_device(wl, dev, n_steps)
    kn_all, vn_all, prio_t = st["k_new"], st["v_new"], st["prio_table"]
    prio_h = host(prio_t)
    rank_o = orc.priority_ranks(prio_h)                 # [nseq, Hkv, n_steps]
    cache = kv.new_decode_cache(nseq, Hkv, D, s, w, k, dtype=torch.bfloat16, device=dev)
    pos_all = torch.arange(n_steps, dtype=torch.int32, device=dev)[:, None].repeat(1, nseq)
    zero_prio = torch.zeros((nseq, Hkv), device=dev)
    prio_steps = prio_t.permute(2, 0, 1).contiguous()   # [n_steps, nseq, Hkv]
    q_fixed = W.make_decode_query_device(wl, dev, 0)
    o = torch.empty((nseq, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nseq, Hq), dtype=torch.float32, device=dev)
    pr = kv.Problem(nseq, Hq, Hkv, 0, D, s, w, k, 0.0, 0, 0)
    n_ws = kv.workspace_size(3, pr)
    ws_raw = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
    ws = ws_raw[(-ws_raw.data_ptr()) % 256:][:n_ws]
    checks = sorted(set(int(c) for c in check_steps if handoff_at <= c < n_steps))
    if handoff_at > 0:
        S = handoff_at
        kp = kn_all[:S].permute(1, 2, 0, 3).contiguous()      # [nseq, Hkv, S, D]
        vp = vn_all[:S].permute(1, 2, 0, 3).contiguous()
        pp = prio_t[:, :, :S].contiguous()
        rank_p, tau_p = kv.thresholds(pp, s, w, k)
        kv.cache_from_prefill(cache, kp, vp, pp, rank_p, tau_p, s, w, k)
        torch.cuda.synchronize()
        held = _held_sets(cache, rank_o, S - 1, s, w, k, Bc)
        n = min(S, Bc)
        sp = cache.slot_pos[:, :, :n].long()
        idx = sp[..., None].expand(-1, -1, -1, D)
        assert torch.equal(cache.k[:, :, :n], torch.gather(kp, 2, idx))
        assert torch.equal(cache.v[:, :, :n], torch.gather(vp, 2, idx))
        canon = orc.canonical_priority(prio_h[:, :, :S])
        sph, sprio = host(cache.slot_pos)[:, :, :n], host(cache.slot_prio)[:, :, :n]
        is_long = (sph >= s) & (sph <= S - 1 - w)
        want_p = np.where(is_long, np.take_along_axis(canon, np.maximum(sph, 0), 2), 0.0)
        assert np.array_equal(sprio.astype(np.float32).view(np.uint32),
                              want_p.astype(np.float32).view(np.uint32))
        ring = host(cache.ring)
        for t in range(max(0, S - w), S):
            j = ring[:, :, t % w]
            assert (np.take_along_axis(sph, j[..., None], 2)[..., 0] == t).all(), t
        del kp, vp, held
    done = 0
    for p in range(handoff_at, n_steps):
        check = done < len(checks) and checks[done] == p
        qd = W.make_decode_query_device(wl, dev, p) if check else q_fixed
        pl = prio_steps[p - w] if p >= w else zero_prio
        kv.decode_step(cache, pos_all[p], qd, kn_all[p], vn_all[p], pl, s, w, k,
                       out_dtype=torch.bfloat16, o=o, lse=lse, ws=ws)
        if not check:
            continue
        done += 1
        torch.cuda.synchronize()
        n = min(p + 1, Bc)
        held = _held_sets(cache, rank_o, p, s, w, k, Bc)
        qh, oh, lh = host(qd), host(o), host(lse)
        for b in out_seqs:
            idx = [held[(b, h)] for h in range(Hkv)]
            kt = np.stack([host(kn_all[torch.as_tensor(idx[h], device=dev), b, h])
                           for h in range(Hkv)])
            vt = np.stack([host(vn_all[torch.as_tensor(idx[h], device=dev), b, h])
                           for h in range(Hkv)])
            local = [np.arange(n)] * Hkv
            oo, ll = orc.decode_attention(qh[b], kt, vt, local)
            ulp = _bf16_half_ulp(np.maximum(np.abs(oo), np.abs(oh[b])))
            assert (np.abs(oh[b] - oo) - ulp).max() <= TOL["bf16"]["o"], (p, b)
            assert np.abs(lh[b] - ll).max() <= TOL["bf16"]["lse"], (p, b)
    assert done == len(checks)


def test_full_decode_b2048():
    """64 sequences, B = 2048, steps 0..5119 (the benchmark times 4096..5119)."""
    wl = W.DECODE_B2048
    announce("full decode 64 x B2048, 5120 steps")
    s, w, Bc = wl.sink, wl.window, wl.budget
    checks = [0, s - 1, s, w - 1, w, w + s, Bc - 1, Bc, Bc + 1, 2 * Bc - 1, 2 * Bc, 4607, 5119]
    _decode_run(wl, 5120, checks, out_seqs=[0, 37, 63])


def test_full_handoff_b2048_then_decode():
    """64 sequences, B = 2048: the cache filled from a 4096-token prompt, as
    the benchmark's decode leg does, then decode steps 4096..4607."""
    wl = W.DECODE_B2048
    announce("full handoff 64 x B2048 from a 4096-token prompt, then 512 steps")
    _decode_run(wl, 4608, [4096, 4097, 4350, 4607], out_seqs=[0, 63], handoff_at=4096)


def test_full_boundary_labels():
    """Teacher boundary labels on the 16k layer's shape (8 KV heads, S = 16384,
    s 16, w 512, k 1520, decay step 64) from seeded stand-in target scores
    whose decay and spread leave the newcomer kept in a mix of rows (about
    35-60 % per head), so both labels occur in every head; sampled rows (the
    first labelled rows, rows around k eligible tokens, random rows and the
    last rows) are compared exactly with the oracle."""
    wl = W.QWEN3_4B_S16K
    announce("full boundary labels 8 x S16384")
    s, w, k, S = wl.sink, wl.window, wl.topk, wl.seq_len
    x = W.make_label_inputs(wl)
    dev = device()
    tb, y = kv.boundary_labels(torch.from_numpy(x["score"]).to(dev),
                               torch.from_numpy(x["log_gamma"]).to(dev), W.LABEL_DECAY_STEP,
                               s, w, k)
    tb, y = host(tb), host(y)
    rng = np.random.default_rng(17)
    rows = sorted(set(list(range(s + w - 3, s + w + 40)) + list(range(s + w + k - 20, s + w + k + 20))
                      + rng.integers(0, S, 400).tolist() + list(range(S - 30, S))))
    want_t, want_y = orc.boundary_labels(x["score"], x["log_gamma"], W.LABEL_DECAY_STEP, s, w, k,
                                         rows=rows)
    assert np.array_equal(tb[..., rows], want_t[..., rows])
    assert np.array_equal(y[..., rows], want_y[..., rows])
    # every row: y in {-1, +1} exactly where a newcomer exists, t_bnd in E(q)
    q = np.arange(S)
    lab = q - w >= s
    assert (y[..., ~lab] == 0).all() and (tb[..., ~lab] == -1).all()
    assert (np.abs(y[..., lab]) == 1).all()
    assert ((tb[..., lab] >= s) & (tb[..., lab] <= (q - w)[lab])).all()
    # a mixed input: both labels in every head, and in the sampled rows too
    kept = (y[..., lab] == 1).mean(axis=-1)[0]
    assert 0.3 <= kept.mean() <= 0.7, kept
    assert ((kept > 0.2) & (kept < 0.8)).all(), kept
    ys = want_y[..., rows]
    assert (ys == 1).sum() > 100 and (ys == -1).sum() > 100


def test_full_masked_bwd_one_kv_head():
    """Backward of the 16k layer (all 32 query / 8 KV heads on the GPU); the
    oracle recomputes KV head 5 and its four query heads in full (every
    element of dq, dk, dv), with the tolerance of the reduced cases."""
    tol = BWD_TOL["bf16"]           # the forward output is bfloat16
    wl = W.QWEN3_4B_S16K
    announce("full masked_attn_bwd 32 x S16384, KV head 5 checked")
    S, s, w, k = wl.seq_len, wl.sink, wl.window, wl.topk
    x = _inputs(wl)
    dev = device()
    dout = W.make_grad_device(wl, dev)
    rank, tau = kv.thresholds(x["prio"], s, w, k)
    o, lse = kv.masked_attn_fwd(x["q"], x["k"], x["v"], rank, tau, s, w, k,
                                out_dtype=torch.bfloat16)
    dq, dk, dv = kv.masked_attn_bwd(x["q"], x["k"], x["v"], o, lse, rank, tau, dout, s, w, k)
    torch.cuda.synchronize()
    h, G = 5, wl.n_q_heads // wl.n_kv_heads
    qs = slice(h * G, (h + 1) * G)
    prio = host(x["prio"][:, h:h + 1])
    rank_o = orc.priority_ranks(prio)
    tau_o = orc.thresholds_by_selection(rank_o, s, w, k)
    rq, rk, rv = orc.masked_attention_backward(host(x["q"][:, qs]), host(x["k"][:, h:h + 1]),
                                               host(x["v"][:, h:h + 1]), rank_o, tau_o, s, w,
                                               host(dout[:, qs]))
    for name, got, ref in (("dq", host(dq[:, qs]), rq), ("dk", host(dk[:, h:h + 1]), rk),
                           ("dv", host(dv[:, h:h + 1]), rv)):
        err = got.astype(np.float64) - ref
        fro = np.linalg.norm(err) / np.linalg.norm(ref)
        mx = np.abs(err).max() / np.abs(ref).max()
        assert fro <= tol["fro"] and mx <= tol["max"], (name, fro, mx)


def test_full_decode_long_131072_steps():
    """8 sequences, B = 4096, decoding to 131072 steps with the constant cache."""
    wl = W.scaled(W.LONG_S128K, batch=8)
    announce("full decode 8 x B4096, 131072 steps")
    Bc = wl.budget
    checks = [Bc - 1, Bc, 2 * Bc, 65535, 131071]
    _decode_run(wl, 131072, checks, out_seqs=[0, 7])
