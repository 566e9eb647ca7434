"""Decode steps and the masked backward replayed from captured HIP graphs give
the eager results.

A decode step takes every input as a device pointer (the position included)
and makes no allocation, copy, memset or host synchronisation, so a model can
capture its per-token loop.  The graph here gathers each step's inputs into
static buffers by a position counter on the device, runs kvpop_decode_step on
two layer caches and advances the counter; every replay is compared bit for bit
with the same steps run eagerly (cache contents, o and LSE), with eager work and
synchronisations between the replays."""
import pytest
import torch

import fixed_budget_sparse_amd as kv
from gpu_util import announce, device

pytestmark = pytest.mark.gpu


def _same_cache(a, b):
    return all(torch.equal(x, y) for x, y in
               ((a.k, b.k), (a.v, b.v), (a.slot_pos, b.slot_pos),
                (a.slot_prio.view(torch.int32), b.slot_prio.view(torch.int32)),
                (a.ring, b.ring), (a.state, b.state)))


@pytest.mark.parametrize("per_graph", [1, 4])
def test_decode_graph_replays_match_eager(per_graph):
    announce(f"decode graph replay, {per_graph} positions per graph")
    dev = device()
    nseq, hq, hkv, D, s, w, k = 2, 8, 2, 128, 4, 16, 40
    n_steps, n_layers = 160, 2
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    qs = torch.randn((n_steps, n_layers, nseq, hq, D), generator=g, device=dev).to(bf)
    kn = torch.randn((n_steps, n_layers, nseq, hkv, D), generator=g, device=dev).to(bf)
    vn = torch.randn((n_steps, n_layers, nseq, hkv, D), generator=g, device=dev).to(bf)
    pr = torch.randn((n_steps, n_layers, nseq, hkv), generator=g, device=dev)
    pr[:w] = 0.0        # no token leaves the window before position w
    pos_all = torch.arange(n_steps, dtype=torch.int32, device=dev)[:, None].repeat(1, nseq)

    # eager reference: o and LSE of every (position, layer)
    ref = [kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=bf, device=dev) for _ in range(n_layers)]
    ref_o = torch.empty((n_steps, n_layers, nseq, hq, D), dtype=bf, device=dev)
    ref_l = torch.empty((n_steps, n_layers, nseq, hq), device=dev)
    for p in range(n_steps):
        for li, c in enumerate(ref):
            kv.decode_step(c, pos_all[p], qs[p, li], kn[p, li], vn[p, li], pr[p, li], s, w, k,
                           out_dtype=bf, o=ref_o[p, li], lse=ref_l[p, li])
    torch.cuda.synchronize()

    caches = [kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=bf, device=dev)
              for _ in range(n_layers)]
    step = torch.zeros(1, dtype=torch.int64, device=dev)
    q_s = torch.empty((1, n_layers, nseq, hq, D), dtype=bf, device=dev)
    kn_s = torch.empty((1, n_layers, nseq, hkv, D), dtype=bf, device=dev)
    vn_s = torch.empty_like(kn_s)
    pr_s = torch.empty((1, n_layers, nseq, hkv), device=dev)
    pos_s = torch.empty((nseq,), dtype=torch.int32, device=dev)
    o_s = torch.empty((n_layers, nseq, hq, D), dtype=bf, device=dev)
    l_s = torch.empty((n_layers, nseq, hq), device=dev)
    prob = kv.Problem(nseq, hq, hkv, 0, D, s, w, k, 0.0, 0, 0)
    n_ws = kv.workspace_size(3, prob)
    ws_raw = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
    ws = ws_raw[(-ws_raw.data_ptr()) % 256:][:n_ws]

    def body(n):
        for _ in range(n):
            torch.index_select(qs, 0, step, out=q_s)
            torch.index_select(kn, 0, step, out=kn_s)
            torch.index_select(vn, 0, step, out=vn_s)
            torch.index_select(pr, 0, step, out=pr_s)
            pos_s.copy_(step.expand(nseq))
            for li, c in enumerate(caches):
                kv.decode_step(c, pos_s, q_s[0, li], kn_s[0, li], vn_s[0, li], pr_s[0, li], s, w,
                               k, out_dtype=bf, o=o_s[li], lse=l_s[li], ws=ws)
            step.add_(1)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        body(1)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body(per_graph)
    for c in caches:
        c.reset()
    step.zero_()
    torch.cuda.synchronize()

    scratch = torch.randn((256, 256), device=dev)
    for r in range(n_steps // per_graph):
        graph.replay()
        # the program's own eager work between replays
        scratch = torch.tanh(scratch @ scratch.t() * 1e-3)
        torch.cuda.synchronize()
        p = (r + 1) * per_graph - 1
        assert int(step.item()) == p + 1, r
        assert torch.equal(o_s, ref_o[p]), (r, p)
        assert torch.equal(l_s.view(torch.int32), ref_l[p].view(torch.int32)), (r, p)
    for a, b in zip(caches, ref):
        assert _same_cache(a, b)


def test_backward_graph_replays_match_eager():
    """The masked backward captured in a HIP graph (its key-major half forked to
    the library's second stream and joined back, as events in the capture)
    replays the eager gradients bit for bit, with eager work between replays."""
    announce("masked backward graph replay (S 1500, split dK/dV tiles)")
    dev = device()
    b, hq, hkv, S, D, s, w, k = 1, 8, 2, 1500, 128, 8, 64, 200
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(91)
    q = torch.randn((b, hq, S, D), generator=g, device=dev).to(bf)
    kk = (torch.randn((b, hkv, S, D), generator=g, device=dev) * 0.3).to(bf)
    v = torch.randn((b, hkv, S, D), generator=g, device=dev).to(bf)
    dout = torch.randn((b, hq, S, D), generator=g, device=dev).to(bf)
    prio = torch.randn((b, hkv, S), generator=g, device=dev)
    rank, tau = kv.thresholds(prio, s, w, k)
    o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf)
    ref = kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k)
    torch.cuda.synchronize()

    f32 = torch.float32
    dq = torch.empty((b, hq, S, D), dtype=f32, device=dev)
    dk = torch.empty((b, hkv, S, D), dtype=f32, device=dev)
    dv = torch.empty((b, hkv, S, D), dtype=f32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k, dq=dq, dk=dk, dv=dv)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k, dq=dq, dk=dk, dv=dv)
    scratch = torch.randn((256, 256), device=dev)
    for r in range(3):
        dq.zero_()
        dk.zero_()
        dv.zero_()
        graph.replay()
        scratch = torch.tanh(scratch @ scratch.t() * 1e-3)
        torch.cuda.synchronize()
        for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (r, name)
