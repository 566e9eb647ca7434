"""Evaluates oracle functions on every row of a large case in worker processes.

The oracle is plain single-threaded NumPy; at the full layer sizes one KV head
takes minutes on one core.  These helpers cut a case into independent slices
(query rows for the forward, tokens for the target), run the unchanged oracle
function on each slice in a pool of spawned worker processes (clean
interpreters that never touch the GPU) and reassemble the result.  Inputs
pass through memory-mapped .npy files in a temporary directory, so workers
share them without copies.  Nothing here computes any part of the method.

Slicing is exact: a row q of the causal forward depends only on keys t <= q,
so a slice of rows [a, b) is evaluated on the first b keys; a token t of the
future target depends on the queries d >= t + w and on key t only.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import tempfile
from typing import Dict

import numpy as np


def n_workers() -> int:
    """Worker processes: the host's CPUs, at most 16 (a GPU machine's share)."""
    return max(1, min(16, os.cpu_count() or 1))


def _load(paths: Dict[str, str]):
    return {k: np.load(p, mmap_mode="r") for k, p in paths.items()}


def _init_worker():
    # one BLAS thread per process: the processes are the parallelism
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _masked_rows(job):
    import oracle as orc
    paths, s, w, a, b = job
    x = _load(paths)
    rows = np.arange(a, b)
    O, L = orc.masked_attention(x["q"][:, :, :b], x["k"][:, :, :b], x["v"][:, :, :b],
                                x["rank"][:, :, :b], x["tau"][:, :, :b], s, w, rows=rows)
    return a, O, L


def _dense_rows(job):
    import oracle as orc
    paths, a, b = job
    x = _load(paths)
    _, L = orc.dense_causal_attention(x["q"][:, :, :b], x["k"][:, :, :b], x["k"][:, :, :b],
                                      rows=np.arange(a, b))
    return a, L


def _target_tokens(job):
    import oracle as orc
    paths, w, ts = job
    x = _load(paths)
    return orc.future_target_eq8(x["q"], x["k"], x["lse"], w, ts=ts)


def _pieces(S: int, n: int):
    """n slices of [0, S) whose sizes shrink towards the end (later rows of a
    causal forward cost more), so the pool's dynamic scheduling balances."""
    edges = np.unique(np.round(S * np.sqrt(np.linspace(0.0, 1.0, n + 1))).astype(int))
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _run(fn, jobs):
    # an executor (not mp.Pool): a worker that dies raises BrokenProcessPool
    # here instead of being replaced silently
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(n_workers(), mp_context=ctx, initializer=_init_worker) as ex:
        return list(ex.map(fn, jobs))


def _save(tmp: str, arrays: Dict[str, np.ndarray]) -> Dict[str, str]:
    paths = {}
    for k, a in arrays.items():
        p = os.path.join(tmp, k + ".npy")
        np.save(p, np.ascontiguousarray(a))
        paths[k] = p
    return paths


def masked_attention_all_rows(q, k, v, rank, tau, s, w):
    """orc.masked_attention on every row (q [b, Hq, S, D], k/v [b, Hkv, S, D],
    rank/tau [b, Hkv, S]); returns O [b, Hq, S, D] and LSE [b, Hq, S]."""
    b, Hq, S, D = q.shape
    with tempfile.TemporaryDirectory() as tmp:
        paths = _save(tmp, {"q": q, "k": k, "v": v, "rank": rank, "tau": tau})
        res = _run(_masked_rows, [(paths, s, w, a, e) for a, e in _pieces(S, 8 * n_workers())])
    O = np.empty((b, Hq, S, D))
    L = np.empty((b, Hq, S))
    for a, o, l in res:
        O[:, :, a:a + o.shape[2]] = o
        L[:, :, a:a + l.shape[2]] = l
    return O, L


def dense_lse_all_rows(q, k):
    """The dense causal (teacher) LSE of every row, [b, Hq, S]."""
    b, Hq, S, D = q.shape
    with tempfile.TemporaryDirectory() as tmp:
        paths = _save(tmp, {"q": q, "k": k})
        res = _run(_dense_rows, [(paths, a, e) for a, e in _pieces(S, 8 * n_workers())])
    L = np.empty((b, Hq, S))
    for a, l in res:
        L[:, :, a:a + l.shape[2]] = l
    return L


def future_target_all_tokens(q, k, lse, w, ts=None):
    """orc.future_target_eq8 on every token (or on the tokens ``ts``):
    q [b, Hq, S, D], k [b, Hkv, S, D], lse [b, Hq, S] -> [b, Hq, len(ts)]."""
    b, Hq, S, D = q.shape
    ts = np.arange(S) if ts is None else np.asarray(ts)
    # interleaved slices: early tokens see the most future queries
    n = min(len(ts), 8 * n_workers())
    slices = [np.arange(i, len(ts), n) for i in range(n)]
    with tempfile.TemporaryDirectory() as tmp:
        paths = _save(tmp, {"q": q, "k": k, "lse": lse})
        res = _run(_target_tokens, [(paths, w, ts[sl]) for sl in slices])
    T = np.empty((b, Hq, len(ts)))
    for sl, t in zip(slices, res):
        T[:, :, sl] = t
    return T
