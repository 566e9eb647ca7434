"""Benchmark of the KVpop fixed-budget sparse hot path on one MI355X.

One step = one pass of the training-side hot path over the Qwen3-4B-shaped
layer (batch 1, 32 query / 8 KV heads, D 128, S 16384, bf16, s 16, w 512,
k 1520, B 2048): kvpop_thresholds -> kvpop_masked_attn_fwd ->
kvpop_future_target (with the dense teacher LSE computed beforehand).
`value` is the algorithmic TFLOP/s of the forward (4 D flop per kept pair) and
the target pass (2 D flop per pair d >= t + w) over the whole step's time.
The decode leg fills a B = 2048 cache of 64 sequences from a 4096-token
prompt (thresholds + kvpop_cache_from_prefill, timed on their own), then times
1024 decode steps (p = 4096..5119) and reports HBM GB/s.

Prints ONE JSON line.  Inputs are synthetic and seeded (workloads.py) and
already resident in HBM when the timed regions start.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E (published)


def fwd_pairs(S, B):
    """kept (q, t) pairs of one head: sum_q min(q + 1, B)."""
    if S <= B:
        return S * (S + 1) // 2
    return B * (B + 1) // 2 + (S - B) * B


def tgt_pairs(S, w):
    n = max(0, S - w)
    return n * (n + 1) // 2


def decode_bytes_per_step(nseq, hq, hkv, D, Bc, esize=2, out_esize=2):
    kv = 2 * nseq * hkv * Bc * D * esize
    q = nseq * hq * D * esize
    o = nseq * hq * D * out_esize
    new = 2 * 2 * nseq * hkv * D * esize       # new K/V read and written
    return kv + q + o + new


def handoff_bytes(nseq, hkv, S, D, s, w, k, esize=2):
    """Algorithmic HBM bytes of one prefill -> decode handoff: the ranks of the
    last row's eligible range, tau, the survivors' priorities, the slot
    metadata and ring written, and min(S, B) K and V rows read and written."""
    Bc = s + w + k
    n = min(S, Bc)
    n_e = max(0, (S - 1 - w) - s + 1)
    per_head = n_e * 4 + 4 + min(k, n_e) * 4 + Bc * 8 + w * 4 + 4 * n * D * esize
    return nseq * hkv * per_head


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration), or
    None when there is none or the kernel's sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.partition(":")
        if sep and key.strip() in ("kernel", "traffic_bytes_per_launch", "sources_sha256", "sources"):
            fields[key.strip()] = val.strip()
    try:
        h = hashlib.sha256()
        for f in fields["sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields["sources_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def sparse_lse_study(kv, torch, q, kk, lse_sparse, tgt, score, s, w, k, eps):
    """The approximate target (the sparse forward's LSE in place of the
    teacher's) against the exact one: how far the target and the score move,
    and how much the kept set of the last row changes when each score serves
    as the priority."""
    S, hkv = q.shape[2], kk.shape[1]
    tgt_sp = kv.future_target(q, kk, lse_sparse, w)
    score_sp = kv.target_score(tgt_sp, hkv, w, eps)
    sel = torch.isfinite(tgt) & (tgt > -20)
    d = (tgt_sp - tgt)[sel].double()
    ds = (score_sp - score)[torch.isfinite(score)].double()
    p = S - 1
    kept = []
    for sc in (score, score_sp):
        rank, tau = kv.thresholds(sc, s, w, k)
        kept.append(rank[:, :, s:p - w + 1] <= tau[:, :, p:p + 1])
    both = (kept[0] & kept[1]).sum(-1).double()
    overlap = both / kept[0].sum(-1).double()
    torch.cuda.synchronize()
    return {"target_diff": {"min": round(d.min().item(), 6), "mean": round(d.mean().item(), 6),
                            "p99": round(torch.quantile(d.float(), 0.99).item(), 6),
                            "max": round(d.max().item(), 6), "n": int(d.numel())},
            "score_diff": {"mean": round(ds.mean().item(), 6), "max": round(ds.abs().max().item(), 6)},
            "last_row_kept_overlap": {"mean": round(overlap.mean().item(), 4),
                                      "min": round(overlap.min().item(), 4)}}


def bench_backward(kv, torch, q, kk, v, o, lse, rank, tau, s, w, k, ev, reps=3, batches=5):
    """Backward of the step's sparse forward (its O and LSE) for a seeded
    upstream gradient dO, the median over `batches` batches of `reps` calls;
    algorithmic work 8 D flop per kept pair per query head (the dP, dQ, dK
    and dV products)."""
    from workloads import QWEN3_4B_S16K, make_grad_device
    dout = make_grad_device(QWEN3_4B_S16K, q.device)
    dq, dk, dv = kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k)
    torch.cuda.synchronize()
    per_batch = []
    for _ in range(batches):
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            kv.masked_attn_bwd(q, kk, v, o, lse, rank, tau, dout, s, w, k, dq=dq, dk=dk, dv=dv)
        e1.record()
        torch.cuda.synchronize()
        per_batch.append(e0.elapsed_time(e1) / reps)
    ms = sorted(per_batch)[len(per_batch) // 2]
    Hq, S, D = q.shape[1], q.shape[2], q.shape[3]
    flop = 8 * D * Hq * fwd_pairs(S, s + w + k)
    return {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2), "flop": flop,
            "frac_mfma_peak": round(flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_labels(kv, torch, score, s, w, k, ev, reps=5):
    """Teacher boundary labels over the step's target score (decay step 64,
    seeded per-head log gamma), timed on their own."""
    from workloads import LABEL_DECAY_STEP, QWEN3_4B_S16K, make_label_inputs
    lg = torch.from_numpy(make_label_inputs(QWEN3_4B_S16K)["log_gamma"]).to(score.device)
    tb, y = kv.boundary_labels(score, lg, LABEL_DECAY_STEP, s, w, k)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        kv.boundary_labels(score, lg, LABEL_DECAY_STEP, s, w, k, t_bnd=tb, y=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    hkv, S = score.shape[1], score.shape[2]
    rows = hkv * max(0, S - s - w)
    kept = (y == 1).sum().item() / max(1, rows)
    return {"ms": round(ms, 4), "decay_step": LABEL_DECAY_STEP, "labelled_rows": rows,
            "rows_per_s": round(rows / (ms * 1e-3), 1), "frac_newcomer_kept": round(kept, 4)}


def bench_tiny(kv, torch, dev, ev, reps=21):
    """The tiny float32 layer (S 512, D 64, 2 query / 1 KV head, s 4, w 32,
    k 64): thresholds, masked forward (float32 MFMA) and future target on the
    teacher LSE, each timed alone (median of `reps`).  Launch-bound at this
    size; reported, not a performance target."""
    from workloads import TINY as wl, make_prefill
    s, w, k, S, D, Hq = wl.sink, wl.window, wl.topk, wl.seq_len, wl.head_dim, wl.n_q_heads
    x = make_prefill(wl)
    q, kk, v, prio = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v", "prio"))
    f32 = torch.float32
    rank_d, tau_d = kv.thresholds(prio, s, w, S)
    _, lse_t = kv.masked_attn_fwd(q, kk, v, rank_d, tau_d, s, w, S, out_dtype=f32)
    rank, tau = kv.thresholds(prio, s, w, k)
    o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=f32)
    tgt = kv.future_target(q, kk, lse_t, w)
    calls = {"thresholds": lambda: kv.thresholds(prio, s, w, k, rank=rank, tau=tau),
             "fwd": lambda: kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=f32, o=o,
                                               lse=lse),
             "target": lambda: kv.future_target(q, kk, lse_t, w, target=tgt)}
    out = {"workload": wl.name, "dtype": "f32", "reps": reps}
    for name, fn in calls.items():
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[name + "_us"] = round(sorted(ts)[len(ts) // 2] * 1e3, 1)
    f_fwd = 4 * D * Hq * fwd_pairs(S, s + w + k)
    f_tgt = 2 * D * Hq * tgt_pairs(S, w)
    out["fwd_flop"], out["target_flop"] = f_fwd, f_tgt
    return out


def bench_layer_c3(kv, torch, dev, ev, reps=5):
    """The Qwen3-8B-shaped layer (S 32768, B 4096): thresholds, masked forward
    and target pass, each timed on its own and end to end (teacher LSE from
    the dense forward beforehand, untimed)."""
    from workloads import QWEN3_8B_S32K as wl, make_prefill_device
    s, w, k, S, D, Hq = wl.sink, wl.window, wl.topk, wl.seq_len, wl.head_dim, wl.n_q_heads
    x = make_prefill_device(wl, dev)
    q, kk, v, prio = x["q"], x["k"], x["v"], x["prio"]
    bf = torch.bfloat16
    rank_d, tau_d = kv.thresholds(prio, s, w, S)
    _, lse_t = kv.masked_attn_fwd(q, kk, v, rank_d, tau_d, s, w, S, out_dtype=bf)
    del rank_d, tau_d
    rank, tau = kv.thresholds(prio, s, w, k)
    o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf)
    tgt = kv.future_target(q, kk, lse_t, w)
    torch.cuda.synchronize()
    t = {"thresholds": [], "fwd": [], "target": [], "end_to_end": []}
    for _ in range(reps):
        e = [ev() for _ in range(4)]
        e[0].record()
        kv.thresholds(prio, s, w, k, rank=rank, tau=tau)
        e[1].record()
        kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf, o=o, lse=lse)
        e[2].record()
        kv.future_target(q, kk, lse_t, w, target=tgt)
        e[3].record()
        torch.cuda.synchronize()
        t["thresholds"].append(e[0].elapsed_time(e[1]))
        t["fwd"].append(e[1].elapsed_time(e[2]))
        t["target"].append(e[2].elapsed_time(e[3]))
        t["end_to_end"].append(e[0].elapsed_time(e[3]))
    # end to end with the target on a second stream beside thresholds +
    # forward, as in the step of the 16k layer
    main_stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    t["overlapped"] = []
    for _ in range(reps):
        e0, e1, done = ev(), ev(), ev()
        e0.record(main_stream)
        side.wait_event(e0)
        with torch.cuda.stream(side):
            kv.future_target(q, kk, lse_t, w, target=tgt)
            done.record(side)
        kv.thresholds(prio, s, w, k, rank=rank, tau=tau)
        kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf, o=o, lse=lse)
        main_stream.wait_event(done)
        e1.record(main_stream)
        torch.cuda.synchronize()
        t["overlapped"].append(e0.elapsed_time(e1))
    med = {n: sorted(v_)[len(v_) // 2] for n, v_ in t.items()}
    f_fwd = 4 * D * Hq * fwd_pairs(S, s + w + k)
    f_tgt = 2 * D * Hq * tgt_pairs(S, w)
    return {"workload": wl.name, "reps": reps, "thresholds_us": round(med["thresholds"] * 1e3, 1),
            "end_to_end_overlapped_ms": round(med["overlapped"], 4),
            "end_to_end_overlapped_tflops":
                round((f_fwd + f_tgt) / (med["overlapped"] * 1e-3) / 1e12, 2),
            "fwd_ms": round(med["fwd"], 4),
            "fwd_tflops": round(f_fwd / (med["fwd"] * 1e-3) / 1e12, 2),
            "target_ms": round(med["target"], 4),
            "target_tflops": round(f_tgt / (med["target"] * 1e-3) / 1e12, 2),
            "end_to_end_ms": round(med["end_to_end"], 4),
            "end_to_end_tflops": round((f_fwd + f_tgt) / (med["end_to_end"] * 1e-3) / 1e12, 2)}


def bench_long_c5(kv, torch, dev, ev, reps=3, n_layers=4):
    """Long context (S 131072, B 4096): thresholds + masked forward of one
    layer; then 8 sequences decoded from position 0 to 131071 over
    `n_layers` independent layer caches in turn (so that no cache is served
    from the last-level cache between its steps), reporting the steady state
    (positions >= B, full caches) and the whole run, and the device memory
    held across the steps."""
    from workloads import LONG_S128K as wl, make_decode_stream_device, make_prefill_device, scaled
    s, w, k, S, D, Hq, Hkv = (wl.sink, wl.window, wl.topk, wl.seq_len, wl.head_dim,
                              wl.n_q_heads, wl.n_kv_heads)
    Bc = s + w + k
    bf = torch.bfloat16
    x = make_prefill_device(wl, dev)
    q, kk, v, prio = x["q"], x["k"], x["v"], x["prio"]
    rank, tau = kv.thresholds(prio, s, w, k)
    o, lse = kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf)
    torch.cuda.synchronize()
    t = {"thresholds": [], "fwd": [], "end_to_end": []}
    for _ in range(reps):
        e = [ev() for _ in range(3)]
        e[0].record()
        kv.thresholds(prio, s, w, k, rank=rank, tau=tau)
        e[1].record()
        kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf, o=o, lse=lse)
        e[2].record()
        torch.cuda.synchronize()
        t["thresholds"].append(e[0].elapsed_time(e[1]))
        t["fwd"].append(e[1].elapsed_time(e[2]))
        t["end_to_end"].append(e[0].elapsed_time(e[2]))
    med = {n: sorted(v_)[len(v_) // 2] for n, v_ in t.items()}
    f_fwd = 4 * D * Hq * fwd_pairs(S, Bc)
    del x, q, kk, v, prio, rank, tau, o, lse
    torch.cuda.empty_cache()

    dwl = scaled(wl, batch=8)
    nseq, n_steps = dwl.batch, S
    st = make_decode_stream_device(dwl, dev, n_steps)
    kn_all, vn_all = st["k_new"], st["v_new"]
    prio_steps = st["prio_table"].permute(2, 0, 1).contiguous()    # [n_steps, nseq, Hkv]
    del st
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    n_q = 1024
    qs = torch.randn((n_q, nseq, Hq, D), generator=g, device=dev).to(bf)
    caches = [kv.new_decode_cache(nseq, Hkv, D, s, w, k, dtype=bf, device=dev)
              for _ in range(n_layers)]
    pos_all = torch.arange(n_steps, dtype=torch.int32, device=dev)[:, None].repeat(1, nseq)
    zero_prio = torch.zeros((nseq, Hkv), device=dev)
    o = torch.empty((nseq, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((nseq, Hq), dtype=torch.float32, device=dev)
    pr = kv.Problem(nseq, Hq, Hkv, 0, D, s, w, k, 0.0, 0, 0)
    n_ws = kv.workspace_size(3, pr)
    ws_raw = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
    ws = ws_raw[(-ws_raw.data_ptr()) % 256:][:n_ws]
    # eager steps: at these sizes the kernels keep the GPU busy (the trace of
    # a step shows no launch gaps), and the inputs are passed by pointer; the
    # step is also capturable in a HIP graph (see the graph replay test)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    mem0 = torch.cuda.memory_allocated(dev)
    e_start, e_full, e_end = ev(), ev(), ev()
    t0 = time.perf_counter()
    e_start.record()
    for p in range(n_steps):
        if p == Bc:
            e_full.record()
        pl = prio_steps[p - w] if p >= w else zero_prio
        for c in caches:
            kv.decode_step(c, pos_all[p], qs[p % n_q], kn_all[p], vn_all[p], pl, s, w, k,
                           out_dtype=bf, o=o, lse=lse, ws=ws)
        if p % 16384 == 16383:
            print(f"[bench] long decode at position {p + 1} of {n_steps}", file=sys.stderr,
                  flush=True)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mem1 = torch.cuda.memory_allocated(dev)
    peak = torch.cuda.max_memory_allocated(dev)
    ms_all = e_start.elapsed_time(e_end)
    ms_full = e_full.elapsed_time(e_end)
    steps_full = n_steps - Bc
    us_layer_step = ms_full * 1e3 / (steps_full * n_layers)
    nbytes = decode_bytes_per_step(nseq, Hq, Hkv, D, Bc)
    gbps = nbytes / (us_layer_step * 1e-6) / 1e9
    cache_bytes = sum(c.k.numel() * 2 * 2 + c.slot_pos.numel() * 8 + c.ring.numel() * 4
                      for c in caches)
    return {"workload": wl.name, "reps": reps,
            "thresholds_us": round(med["thresholds"] * 1e3, 1),
            "fwd_ms": round(med["fwd"], 4),
            "fwd_tflops": round(f_fwd / (med["fwd"] * 1e-3) / 1e12, 2),
            "end_to_end_ms": round(med["end_to_end"], 4),
            "decode": {"sequences": nseq, "positions": [0, n_steps - 1], "layer_caches": n_layers,
                       "steady_state": {"positions": [Bc, n_steps - 1],
                                        "us_per_layer_step": round(us_layer_step, 2),
                                        "bytes_per_layer_step": nbytes,
                                        "GB/s": round(gbps, 1),
                                        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)},
                       "all_steps": {"ms": round(ms_all, 1), "wall_s": round(wall, 2),
                                     "tokens_per_s_per_layer":
                                         round(nseq * n_steps / (ms_all * 1e-3), 1)},
                       "device_memory": {"caches_bytes": cache_bytes,
                                         "allocated_before": mem0, "allocated_after": mem1,
                                         "peak_during": peak}}}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 20 untimed steps bring the chip to its sustained clock: with 3, the
    # first ten or so timed steps ran about 7 % slower than the rest
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the S 32768 layer and the S 131072 long-context legs")
    ap.add_argument("--overlap", choices=("full", "forward", "thresholds", "none"), default="full",
                    help="full: the target on a second stream beside thresholds + forward; "
                         "forward: the thresholds alone, then the target beside the forward; "
                         "thresholds: beside the thresholds only, the forward after it; "
                         "none: the three in order on one stream")
    ap.add_argument("--no-isolated", dest="isolated", action="store_false",
                    help="skip the forward and target timed alone after the step")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def host_description():
    """The host the oracle runs on: CPU model, logical CPUs, NumPy's BLAS."""
    info = {"nproc": os.cpu_count()}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = {k: blas[0].get(k) for k in ("internal_api", "version", "num_threads",
                                                        "threading_layer", "architecture")}
    except Exception:  # pragma: no cover
        pass
    return info


def cpu_baseline(x, s, w, k):
    """The oracle as it stands (float64 NumPy, one process) timed on the host
    on a bounded sample of every workload, pass by pass (about 20 s of CPU
    work): the tiny float32 layer in full; the 16k and 32k layers, the
    long-context layer and the 64-sequence decode on stated samples.  Each
    pass reports its algorithmic work and rate; `value` is the 16k layer's
    forward + target sample (the headline metric's unit)."""
    import numpy as np
    import oracle as orc
    import workloads as W
    host = host_description()
    cores = int((host.get("blas") or {}).get("num_threads") or 1)
    passes = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    def rate(flop, secs):
        return round(flop / secs / 1e12, 6)

    def prefill(wl, x_, rows_fwd, ts_tgt, label, target=True):
        S_, D_, Hq_ = x_["q"].shape[2], x_["q"].shape[3], x_["q"].shape[1]
        s_, w_, k_ = wl.sink, wl.window, wl.topk
        B_ = s_ + w_ + k_
        thr_rows = np.arange(S_) if S_ <= 16384 else np.linspace(0, S_ - 1, 2048).astype(np.int64)
        (rank, _), t_rank = timed(lambda: (orc.priority_ranks(x_["prio"]), None))
        tau_s, t_tau = timed(lambda: orc.thresholds_by_selection(rank, s_, w_, k_, rows=thr_rows))
        tau = np.zeros(rank.shape, np.int64)
        tau[..., thr_rows] = tau_s
        if S_ > 16384:            # the forward's rows need their own cutoffs
            tau[..., rows_fwd] = orc.thresholds_by_selection(rank, s_, w_, k_, rows=rows_fwd)
        _, t_fwd = timed(lambda: orc.masked_attention(x_["q"], x_["k"], x_["v"], rank, tau, s_, w_,
                                                      rows=rows_fwd))
        f_fwd = 4 * D_ * Hq_ * sum(min(int(r) + 1, B_) for r in rows_fwd)
        out = {"thresholds": {"rows": len(thr_rows), "seconds": round(t_rank + t_tau, 3),
                              "rows_per_s": round(len(thr_rows) / (t_rank + t_tau), 1)},
               "masked_fwd": {"rows": len(rows_fwd), "heads": Hq_, "seconds": round(t_fwd, 3),
                              "flop": f_fwd, "TFLOP/s": rate(f_fwd, t_fwd)}}
        if target:
            # the teacher LSE of the rows the sampled tokens need (untimed)
            need = np.arange(int(min(ts_tgt)) + w_, S_)
            lse = np.zeros((1, Hq_, S_))
            _, lse[:, :, need] = orc.dense_causal_attention(x_["q"], x_["k"], x_["k"], rows=need,
                                                           block=512)
            _, t_tgt = timed(lambda: orc.future_target_eq8(x_["q"], x_["k"], lse, w_, ts=ts_tgt))
            f_tgt = 2 * D_ * Hq_ * sum(max(0, S_ - int(t) - w_) for t in ts_tgt)
            out["future_target"] = {"tokens": len(ts_tgt), "heads": Hq_, "seconds": round(t_tgt, 3),
                                    "flop": f_tgt, "TFLOP/s": rate(f_tgt, t_tgt)}
        passes[label] = out
        return out

    # tiny float32 layer: every row and token
    xt = W.make_prefill(W.TINY)
    St = W.TINY.seq_len
    prefill(W.TINY, xt, np.arange(St), np.arange(St - W.TINY.window), W.TINY.name)
    # 16k layer (the step's inputs): 1536 forward rows, 1024 target tokens
    # among the last 2048 that have future queries
    S = x["q"].shape[2]
    r16 = prefill(W.QWEN3_4B_S16K, x, np.linspace(0, S - 1, 1536).astype(np.int64),
                  np.linspace(S - w - 2048, S - 1 - w, 1024).astype(np.int64), W.QWEN3_4B_S16K.name)
    # 32k layer and long context: one KV head with its 4 query heads (the same
    # recipe), cutoffs of 2048 sampled rows, 576 / 144 forward rows
    for wl_, nrows in ((W.QWEN3_8B_S32K, 576), (W.LONG_S128K, 144)):
        one = W.scaled(wl_, n_q_heads=wl_.group, n_kv_heads=1)
        xs = W.make_prefill(one)
        Sx = one.seq_len
        prefill(one, xs, np.linspace(0, Sx - 1, nrows).astype(np.int64), None,
                wl_.name + " (one KV head)", target=False)
        del xs
    # decode: one (sequence, KV head) simulated over 3072 positions (the cache
    # fills at 2048), and the attention of one sequence's 32 query heads at 96
    # of those steps
    wd = W.DECODE_B2048
    n_steps, D, Hq, Hkv = 3072, wd.head_dim, wd.n_q_heads, wd.n_kv_heads
    table = W.make_decode_prio_table(wd, n_tokens=n_steps, batch=1)
    _, t_sim = timed(lambda: orc.decode_simulate(table[0, 0], wd.sink, wd.window, wd.topk,
                                                 n_steps, record=[]))
    rng = np.random.default_rng(7)
    kt = rng.standard_normal((Hkv, n_steps, D)).astype(np.float32)
    vt = rng.standard_normal((Hkv, n_steps, D)).astype(np.float32)
    steps = np.linspace(wd.budget, n_steps - 1, 96).astype(int)
    held, _ = orc.decode_simulate(table[0, 0], wd.sink, wd.window, wd.topk, n_steps, record=steps)
    qd = rng.standard_normal((Hq, D)).astype(np.float32)
    _, t_att = timed(lambda: [orc.decode_attention(qd, kt, vt, [held[p]] * Hkv) for p in steps])
    bytes_att = 2 * Hkv * wd.budget * D * 2 * len(steps)
    passes[wd.name] = {"membership": {"positions": n_steps, "seconds": round(t_sim, 3),
                                      "steps_per_s": round(n_steps / t_sim, 1)},
                       "attention": {"steps": len(steps), "sequences": 1, "seconds": round(t_att, 3),
                                     "cache_bytes": bytes_att,
                                     "GB/s": round(bytes_att / t_att / 1e9, 4)}}
    f16 = r16["masked_fwd"]["flop"] + r16["future_target"]["flop"]
    t16 = r16["masked_fwd"]["seconds"] + r16["future_target"]["seconds"]
    total = sum(v["seconds"] for p in passes.values() for v in p.values())
    return {"value": f16 / t16 / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "16k layer: masked forward on 1536 rows x 32 heads and future target on 1024 "
                      "tokens x 32 heads (teacher LSE untimed); every pass of every workload in "
                      f"`passes`; {total:.1f} s of CPU work in all",
            "precision": "float64 (the oracle's arithmetic)", "host": host, "passes": passes,
            "seconds": round(total, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU, which holds every KV head of the layer; run with --gpus 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import fixed_budget_sparse_amd as kv
    from workloads import DECODE_B2048, QWEN3_4B_S16K, make_prefill

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = QWEN3_4B_S16K
    s, w, k, S, D, Hq, Hkv = wl.sink, wl.window, wl.topk, wl.seq_len, wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    x = make_prefill(wl)
    bf = torch.bfloat16
    q = torch.from_numpy(x["q"]).to(bf).to(dev)
    kk = torch.from_numpy(x["k"]).to(bf).to(dev)
    v = torch.from_numpy(x["v"]).to(bf).to(dev)
    prio = torch.from_numpy(x["prio"]).to(dev)
    rank = torch.empty(prio.shape, dtype=torch.int32, device=dev)
    tau = torch.empty_like(rank)
    o = torch.empty(q.shape, dtype=bf, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    tgt = torch.empty_like(lse)
    # teacher (dense causal) LSE: the forward with k >= S, untimed
    rank_d, tau_d = kv.thresholds(prio, s, w, S)
    _, lse_teacher = kv.masked_attn_fwd(q, kk, v, rank_d, tau_d, s, w, S, out_dtype=bf)
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        src.copy_(torch.ones_like(src))
        dst = src.clone()
        del src, dst
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    times = {"thr": [], "fwd": [], "tgt": []}
    # The target pass reads only Q, K and the teacher LSE, so it does not wait
    # for the cutoffs or the forward: it runs on a second stream (default
    # priority) beside them, and the step ends when both streams are done.
    # The cutoff kernels fill only a few CUs; the target fills the rest.
    main_stream = torch.cuda.current_stream(dev)
    tgt_stream = torch.cuda.Stream(dev) if args.overlap != "none" else main_stream

    def one_step(record):
        e0, e1, e2, e3, e4, e5, e6 = ev(), ev(), ev(), ev(), ev(), ev(), ev()
        def target():
            with torch.cuda.stream(tgt_stream):
                e4.record(tgt_stream)
                kv.future_target(q, kk, lse_teacher, w, target=tgt)
                e5.record(tgt_stream)

        e0.record(main_stream)
        if args.overlap in ("full", "thresholds"):
            tgt_stream.wait_event(e0)
            target()
        kv.thresholds(prio, s, w, k, rank=rank, tau=tau)
        e1.record(main_stream)
        if args.overlap == "forward":
            tgt_stream.wait_event(e1)
            target()
        if args.overlap == "thresholds":
            main_stream.wait_event(e5)   # the forward runs after the target
        e6.record(main_stream)
        kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf, o=o, lse=lse)
        e2.record(main_stream)
        if args.overlap in ("full", "forward"):
            main_stream.wait_event(e5)
        elif args.overlap == "none":
            target()
        e3.record(main_stream)
        if record is not None:
            record.append((e0, e1, e2, e3, e4, e5, e6))

    for _ in range(args.warmup):
        one_step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ev = []
    for e0, e1, e2, e3, e4, e5, e6 in recs:
        times["thr"].append(e0.elapsed_time(e1))
        times["fwd"].append(e6.elapsed_time(e2))
        times["tgt"].append(e4.elapsed_time(e5))
        step_ev.append(e0.elapsed_time(e3))
    ms_step = wall * 1e3 / args.steps
    # after the timed region: the forward and the target each alone on the
    # chip (in the step they share it): 7 batches of 10 back-to-back calls,
    # the median batch's time per call
    iso = {}
    alone = (("fwd", lambda: kv.masked_attn_fwd(q, kk, v, rank, tau, s, w, k, out_dtype=bf,
                                                o=o, lse=lse)),
             ("tgt", lambda: kv.future_target(q, kk, lse_teacher, w, target=tgt)))
    for name, fn in alone if args.isolated else ():
        fn()
        per = []
        for _ in range(7):
            ea, eb = ev(), ev()
            ea.record()
            for _ in range(10):
                fn()
            eb.record()
            torch.cuda.synchronize()
            per.append(ea.elapsed_time(eb) / 10)
        iso[name] = sorted(per)[len(per) // 2]
    # the target score per KV head, timed alone, then the sparse-LSE study
    # (untimed): `lse` holds the last step's sparse LSE, `tgt` the exact target
    eps = 1e-6
    score = torch.empty((1, Hkv, S), dtype=torch.float32, device=dev)
    kv.target_score(tgt, Hkv, w, eps, score=score)
    torch.cuda.synchronize()
    es, ee = ev(), ev()
    es.record()
    for _ in range(20):
        kv.target_score(tgt, Hkv, w, eps, score=score)
    ee.record()
    torch.cuda.synchronize()
    score_us = es.elapsed_time(ee) * 1e3 / 20
    study = sparse_lse_study(kv, torch, q, kk, lse, tgt, score, s, w, k, eps)
    labels = bench_labels(kv, torch, score, s, w, k, ev)
    backward = bench_backward(kv, torch, q, kk, v, o, lse, rank, tau, s, w, k, ev)
    B = s + w + k
    f_fwd = 4 * D * Hq * fwd_pairs(S, B)
    f_tgt = 2 * D * Hq * tgt_pairs(S, w)
    avg = {n: sum(t) / len(t) for n, t in times.items()}
    med = {n: sorted(t)[len(t) // 2] for n, t in times.items()}
    value = (f_fwd + f_tgt) / (ms_step * 1e-3) / 1e12
    tgt_tflops = f_tgt / (avg["tgt"] * 1e-3) / 1e12
    fwd_tflops = f_fwd / (avg["fwd"] * 1e-3) / 1e12

    out = {
        "metric": "masked fwd+target TFLOP/s (%MFMA peak) S=16k; decode GB/s (%HBM) at B=2048",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "seq_len": S, "sink": s, "window": w, "topk": k, "budget": B,
                   "step": {"full": "thresholds + masked fwd, future target on a second "
                                    "stream beside them",
                            "forward": "thresholds, then masked fwd with the future target "
                                       "on a second stream beside it",
                            "thresholds": "future target on a second stream beside the "
                                          "thresholds, then the masked fwd",
                            "none": "thresholds + masked fwd + future target"}[args.overlap],
                   "decode_workload": DECODE_B2048.name},
        "frac_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels_ms": {n: round(t, 4) for n, t in avg.items()},
        "kernels_ms_median": {n: round(t, 4) for n, t in med.items()},
        "step_ms_events": round(sum(step_ev) / len(step_ev), 4),
        "step_ms_median": round(sorted(step_ev)[len(step_ev) // 2], 4),
        "isolated_ms": {n: round(t, 4) for n, t in iso.items()} or None,
        "isolated_tflops": {"fwd": round(f_fwd / (iso["fwd"] * 1e-3) / 1e12, 2),
                            "tgt": round(f_tgt / (iso["tgt"] * 1e-3) / 1e12, 2)} if iso else None,
        "fwd_tflops": round(fwd_tflops, 2),
        "target_tflops": round(tgt_tflops, 2),
        "roofline": {"bound": "mfma", "kernel": "future_target_kernel",
                     "achieved": round(tgt_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tgt_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("future_target", "qwen3-4b-S16384"),
                     "traffic_unit": "bytes/launch"},
        "target_score": {"us": round(score_us, 2), "eps": eps,
                         "bytes": 4 * (Hq + Hkv) * S,
                         "GB/s": round(4 * (Hq + Hkv) * S / (score_us * 1e-6) / 1e9, 1)},
        "sparse_lse_study": study,
        "boundary_labels": labels,
        "backward": backward,
    }

    if not args.no_decode:
        out["decode"] = bench_decode(kv, torch, np, dev, args.decode_steps)
    # every hot kernel against its roofline, from launches alone on the chip:
    # the forward and target calls (7 x 10 launches, median), the decode step
    # (1024 steps) and the backward (3 calls)
    rl = {}
    if iso:
        for name, flop, kern in (("masked_fwd", f_fwd, ["key_end_kernel", "tile_list_kernel",
                                                        "masked_fwd_kernel"]),
                                 ("future_target", f_tgt, ["future_target_kernel"])):
            ms = iso["fwd" if name == "masked_fwd" else "tgt"]
            ach = flop / (ms * 1e-3) / 1e12
            rl[name] = {"bound": "mfma", "kernels": kern, "ms_per_call": round(ms, 4),
                        "algorithmic": flop, "achieved": round(ach, 2),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    if "decode" in out:
        dd = out["decode"]
        rl["decode_step"] = {"bound": "hbm", "kernels": ["decode_attend_kernel"],
                             "us_per_call": dd["us_per_step"], "algorithmic": dd["bytes_per_step"],
                             "achieved": dd["GB/s"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": dd["frac_hbm_peak"], "traffic": dd["traffic"]}
    # (the key-major kernels run on the library's second stream; the call's
    # time spans both)
    rl["masked_bwd"] = {"bound": "mfma", "kernels": ["key_end_kernel", "tile_list_kernel",
                                                     "bwd_dot_kernel", "bwd_dq_kernel",
                                                     "bwd_key_order_kernel", "bwd_tile_plan_kernel",
                                                     "bwd_dkdv_kernel", "bwd_dkdv_merge_kernel"],
                        "ms_per_call": backward["ms"], "algorithmic": backward["flop"],
                        "achieved": backward["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": backward["frac_mfma_peak"]}
    out["rooflines"] = rl
    if not args.no_other_configs:
        del q, kk, v, o, lse, tgt, lse_teacher, rank_d, tau_d
        torch.cuda.empty_cache()
        out["other_configs"] = {"tiny": bench_tiny(kv, torch, dev, ev),
                                "qwen3-8b-layer": bench_layer_c3(kv, torch, dev, ev),
                                "long-context": bench_long_c5(kv, torch, dev, ev)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, s, w, k)
    print(json.dumps(out))


def bench_decode(kv, torch, np, dev, n_timed):
    from workloads import DECODE_B2048 as wl
    s, w, k, D, Hq, Hkv, nseq = wl.sink, wl.window, wl.topk, wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.batch
    Bc = s + w + k
    bf = torch.bfloat16
    p_start = 2 * Bc                      # 4096: cache full, ~2k tokens already evicted
    p_end = p_start + n_timed
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    prio_table = torch.randn((nseq, Hkv, p_end), generator=g, device=dev)
    cache = kv.new_decode_cache(nseq, Hkv, D, s, w, k, dtype=bf, device=dev)
    o = torch.empty((nseq, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((nseq, Hq), dtype=torch.float32, device=dev)
    pos_all = torch.arange(p_end, dtype=torch.int32, device=dev)[:, None].repeat(1, nseq).contiguous()
    zero_prio = torch.zeros((nseq, Hkv), device=dev)
    pr = kv.Problem(nseq, Hq, Hkv, 0, D, s, w, k, 0.0, 0, 0)
    n_ws = kv.workspace_size(3, pr)
    ws = torch.empty(n_ws + 256, dtype=torch.uint8, device=dev)
    ws = ws[(-ws.data_ptr()) % 256:][:n_ws]

    def prio_at(p):
        u = p - w
        return prio_table[:, :, u].contiguous() if u >= 0 else zero_prio

    # the cache after a prompt of p_start tokens: thresholds over the prompt's
    # priorities, then the handoff of the last row's kept set (timed apart;
    # the handoff rewrites the whole cache, so repeats are idempotent)
    kp = torch.randn((nseq, Hkv, p_start, D), generator=g, device=dev).to(bf)
    vp = torch.randn((nseq, Hkv, p_start, D), generator=g, device=dev).to(bf)
    prio_prompt = prio_table[:, :, :p_start].contiguous()
    rank_p = torch.empty(prio_prompt.shape, dtype=torch.int32, device=dev)
    tau_p = torch.empty_like(rank_p)
    ho_ms = {"thresholds": [], "cache_from_prefill": []}
    for rep in range(12):
        a, b_, c_ = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record()
        kv.thresholds(prio_prompt, s, w, k, rank=rank_p, tau=tau_p)
        b_.record()
        kv.cache_from_prefill(cache, kp, vp, prio_prompt, rank_p, tau_p, s, w, k)
        c_.record()
        torch.cuda.synchronize()
        if rep >= 2:
            ho_ms["thresholds"].append(a.elapsed_time(b_))
            ho_ms["cache_from_prefill"].append(b_.elapsed_time(c_))
    ho_avg = {n: sum(t) / len(t) for n, t in ho_ms.items()}
    ho_bytes = handoff_bytes(nseq, Hkv, p_start, D, s, w, k)
    del kp, vp
    # pre-drawn inputs of the timed steps, resident in HBM
    qs = torch.randn((n_timed, nseq, Hq, D), generator=g, device=dev).to(bf)
    kns = torch.randn((n_timed, nseq, Hkv, D), generator=g, device=dev).to(bf)
    vns = torch.randn((n_timed, nseq, Hkv, D), generator=g, device=dev).to(bf)
    pls = torch.stack([prio_at(p) for p in range(p_start, p_end)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(n_timed):
        kv.decode_step(cache, pos_all[p_start + i], qs[i], kns[i], vns[i], pls[i], s, w, k,
                       out_dtype=bf, o=o, lse=lse, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    us_step = ms * 1e3 / n_timed
    nbytes = decode_bytes_per_step(nseq, Hq, Hkv, D, Bc)
    gbps = nbytes / (us_step * 1e-6) / 1e9
    traffic = measured_traffic("decode_attend", wl.name)
    return {"workload": wl.name, "steps_timed": n_timed, "positions": [p_start, p_end - 1],
            "us_per_step": round(us_step, 2), "wall_us_per_step": round(wall * 1e6 / n_timed, 2),
            "bytes_per_step": nbytes, "GB/s": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            # DRAM bytes per step from the committed counter summary (None once
            # the kernel's sources change): the algorithmic bytes plus the slot
            # metadata the step reads
            "traffic": traffic,
            "traffic_GB/s": round(traffic / (us_step * 1e-6) / 1e9, 1) if traffic else None,
            "tokens_per_s": round(nseq / (us_step * 1e-6), 1),
            "handoff": {"prompt_tokens": p_start,
                        "thresholds_ms": round(ho_avg["thresholds"], 4),
                        "cache_from_prefill_ms": round(ho_avg["cache_from_prefill"], 4),
                        "cache_from_prefill_bytes": ho_bytes,
                        "cache_from_prefill_GB/s":
                            round(ho_bytes / (ho_avg["cache_from_prefill"] * 1e-3) / 1e9, 1)}}


if __name__ == "__main__":
    main()
