"""ctypes binding of the libkvpop C ABI (include/kvpop.h).

Each function checks tensor devices, dtypes, shapes and contiguity, allocates
outputs and the workspace with PyTorch (device memory only), passes raw
pointers and the current HIP stream to the library, and raises KvpopError on a
non-zero status.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvpop.so")

KVPOP_BF16, KVPOP_F32 = 0, 1
CALL_THRESHOLDS, CALL_MASKED_FWD, CALL_FUTURE_TARGET, CALL_DECODE = 0, 1, 2, 3
CALL_CACHE_FROM_PREFILL, CALL_TARGET_SCORE, CALL_BOUNDARY_LABELS, CALL_MASKED_BWD = 4, 5, 6, 7

EXPORTED_SYMBOLS = (
    "kvpop_workspace_size",
    "kvpop_thresholds",
    "kvpop_masked_attn_fwd",
    "kvpop_future_target",
    "kvpop_decode_step",
    "kvpop_decode_step_noalloc",
    "kvpop_cache_from_prefill",
    "kvpop_target_score",
    "kvpop_boundary_labels",
    "kvpop_masked_attn_bwd",
    "kvpop_status_string",
    "kvpop_abi_version",
    "kvpop_debug_reverse_launch_order",
)


class KvpopError(RuntimeError):
    """A libkvpop call returned a non-zero status, or the library is unusable."""


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("window", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("qkv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("slot_pos", ctypes.c_void_p),
                ("slot_prio", ctypes.c_void_p), ("ring", ctypes.c_void_p),
                ("state", ctypes.c_void_p)]


CACHE_STATE_WORDS = 8   # KVPOP_CACHE_STATE_WORDS


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libkvpop.so (after torch, so the HIP runtime torch loaded is reused)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise KvpopError(f"{_LIB_PATH} is not built: run `python -m fixed_budget_sparse_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.kvpop_workspace_size.argtypes = [ctypes.c_int32, P]
        L.kvpop_workspace_size.restype = sz
        L.kvpop_thresholds.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.kvpop_masked_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.kvpop_future_target.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.kvpop_decode_step.argtypes = [P, ctypes.POINTER(_Cache), vp, vp, vp, vp, vp, vp, vp,
                                        vp, sz, vp]
        L.kvpop_decode_step_noalloc.argtypes = [P, ctypes.POINTER(_Cache), vp, vp, vp, vp, vp,
                                                vp, vp, vp]
        L.kvpop_cache_from_prefill.argtypes = [P, ctypes.POINTER(_Cache), vp, vp, vp, vp, vp, vp]
        L.kvpop_target_score.argtypes = [P, vp, ctypes.c_float, vp, vp]
        L.kvpop_boundary_labels.argtypes = [P, vp, vp, ctypes.c_int32, vp, vp, vp]
        L.kvpop_masked_attn_bwd.argtypes = [P] + [vp] * 12 + [sz, vp]
        for f in ("kvpop_thresholds", "kvpop_masked_attn_fwd", "kvpop_future_target",
                  "kvpop_decode_step", "kvpop_decode_step_noalloc", "kvpop_cache_from_prefill", "kvpop_target_score",
                  "kvpop_boundary_labels", "kvpop_masked_attn_bwd"):
            getattr(L, f).restype = ctypes.c_int
        L.kvpop_status_string.argtypes = [ctypes.c_int]
        L.kvpop_status_string.restype = ctypes.c_char_p
        L.kvpop_abi_version.argtypes = []
        L.kvpop_abi_version.restype = ctypes.c_int32
        L.kvpop_debug_reverse_launch_order.argtypes = [ctypes.c_int32]
        L.kvpop_debug_reverse_launch_order.restype = None
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().kvpop_abi_version())


def debug_reverse_launch_order(on: bool) -> None:
    """Testing aid: launch the forward's, target's and backward's workgroups
    last tile first (outputs must not change)."""
    lib().kvpop_debug_reverse_launch_order(1 if on else 0)


@dataclasses.dataclass
class Problem:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    sink: int
    window: int
    topk: int
    softmax_scale: float = 0.0
    qkv_dtype: int = KVPOP_BF16
    out_dtype: int = KVPOP_F32

    def c(self) -> _Problem:
        return _Problem(self.batch, self.n_q_heads, self.n_kv_heads, self.seq_len, self.head_dim,
                        self.sink, self.window, self.topk, self.softmax_scale, self.qkv_dtype,
                        self.out_dtype)


def workspace_size(call: int, pr: Problem) -> int:
    c = pr.c()
    return int(lib().kvpop_workspace_size(call, ctypes.byref(c)))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KVPOP_BF16
    if dt == torch.float32:
        return KVPOP_F32
    raise KvpopError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise KvpopError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise KvpopError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise KvpopError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise KvpopError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise KvpopError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise KvpopError(f"{name} must be contiguous")


def _vp(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(call: int, pr: Problem, device) -> Tuple[Optional[torch.Tensor], int]:
    n = workspace_size(call, pr)
    if n == 0:
        return None, 0
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n], n


def _status(st: int, what: str):
    if st != 0:
        msg = lib().kvpop_status_string(st).decode()
        raise KvpopError(f"{what} failed: status {st} ({msg})")


def thresholds(prio: torch.Tensor, sink: int, window: int, topk: int,
               rank: Optional[torch.Tensor] = None, tau: Optional[torch.Tensor] = None):
    """rank, tau = thresholds(prio[b, Hkv, S] float32, s, w, k)."""
    b, hkv, S = prio.shape
    dev = prio.device
    _need(prio, "prio", (b, hkv, S), torch.float32)
    rank = torch.empty((b, hkv, S), dtype=torch.int32, device=dev) if rank is None else rank
    tau = torch.empty((b, hkv, S), dtype=torch.int32, device=dev) if tau is None else tau
    _need(rank, "rank", (b, hkv, S), torch.int32, dev)
    _need(tau, "tau", (b, hkv, S), torch.int32, dev)
    pr = Problem(b, hkv, hkv, S, 128, sink, window, topk)
    ws, n = _workspace(CALL_THRESHOLDS, pr, dev)
    c = pr.c()
    _status(lib().kvpop_thresholds(ctypes.byref(c), _vp(prio), _vp(rank), _vp(tau), _vp(ws), n,
                                   _stream(dev)), "kvpop_thresholds")
    return rank, tau


def masked_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rank: torch.Tensor,
                    tau: torch.Tensor, sink: int, window: int, topk: int,
                    softmax_scale: float = 0.0, out_dtype: torch.dtype = torch.float32,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """o, lse = masked_attn_fwd(q[b,Hq,S,D], k, v [b,Hkv,S,D], rank, tau, s, w, k)."""
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    dev = q.device
    _need(q, "q", (b, hq, S, D), q.dtype)
    _need(k, "k", (b, hkv, S, D), q.dtype, dev)
    _need(v, "v", (b, hkv, S, D), q.dtype, dev)
    _need(rank, "rank", (b, hkv, S), torch.int32, dev)
    _need(tau, "tau", (b, hkv, S), torch.int32, dev)
    o = torch.empty((b, hq, S, D), dtype=out_dtype, device=dev) if o is None else o
    lse = torch.empty((b, hq, S), dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (b, hq, S, D), out_dtype, dev)
    _need(lse, "lse", (b, hq, S), torch.float32, dev)
    pr = Problem(b, hq, hkv, S, D, sink, window, topk, softmax_scale, _dtype_code(q.dtype),
                 _dtype_code(out_dtype))
    ws, n = _workspace(CALL_MASKED_FWD, pr, dev)
    c = pr.c()
    _status(lib().kvpop_masked_attn_fwd(ctypes.byref(c), _vp(q), _vp(k), _vp(v), _vp(rank),
                                        _vp(tau), _vp(o), _vp(lse), _vp(ws), n, _stream(dev)),
            "kvpop_masked_attn_fwd")
    return o, lse


def future_target(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, window: int,
                  softmax_scale: float = 0.0, target: Optional[torch.Tensor] = None):
    """target[b,Hq,S] = ln sum_{d>=t+w} exp(scale <q_d,k_t> - lse_d)."""
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    dev = q.device
    _need(q, "q", (b, hq, S, D), q.dtype)
    _need(k, "k", (b, hkv, S, D), q.dtype, dev)
    _need(lse, "lse", (b, hq, S), torch.float32, dev)
    target = torch.empty((b, hq, S), dtype=torch.float32, device=dev) if target is None else target
    _need(target, "target", (b, hq, S), torch.float32, dev)
    pr = Problem(b, hq, hkv, S, D, 0, window, 0, softmax_scale, _dtype_code(q.dtype), KVPOP_F32)
    ws, n = _workspace(CALL_FUTURE_TARGET, pr, dev)
    c = pr.c()
    _status(lib().kvpop_future_target(ctypes.byref(c), _vp(q), _vp(k), _vp(lse), _vp(target),
                                      _vp(ws), n, _stream(dev)), "kvpop_future_target")
    return target


@dataclasses.dataclass
class DecodeCache:
    """Caller-owned decode cache arrays (see kvpop_cache in include/kvpop.h)."""
    k: torch.Tensor          # [b, Hkv, Bc, D]
    v: torch.Tensor          # [b, Hkv, Bc, D]
    slot_pos: torch.Tensor   # [b, Hkv, Bc] int32
    slot_prio: torch.Tensor  # [b, Hkv, Bc] float32
    ring: torch.Tensor       # [b, Hkv, w] int32
    # [b, Hkv, CACHE_STATE_WORDS] int32: the next step's record, or None (every
    # full step then scans the slots)
    state: Optional[torch.Tensor] = None

    def c(self) -> _Cache:
        return _Cache(self.k.data_ptr(), self.v.data_ptr(), self.slot_pos.data_ptr(),
                      self.slot_prio.data_ptr(), self.ring.data_ptr(),
                      self.state.data_ptr() if self.state is not None else None)

    def reset(self) -> None:
        """Back to the empty state of new_decode_cache, in place (same memory)."""
        self.k.zero_()
        self.v.zero_()
        self.slot_pos.fill_(-1)
        self.slot_prio.zero_()
        self.ring.zero_()
        if self.state is not None:
            self.state.zero_()

    def arrays(self):
        """Every array of the cache (the state included when present)."""
        return tuple(t for t in (self.k, self.v, self.slot_pos, self.slot_prio, self.ring,
                                 self.state) if t is not None)

    def clone(self) -> "DecodeCache":
        return DecodeCache(*(t.clone() if t is not None else None
                             for t in (self.k, self.v, self.slot_pos, self.slot_prio,
                                       self.ring, self.state)))

    def check(self, b: int, hkv: int, Bc: int, D: int, window: int, dtype, dev) -> None:
        _need(self.k, "cache.k", (b, hkv, Bc, D), dtype, dev)
        _need(self.v, "cache.v", (b, hkv, Bc, D), dtype, dev)
        _need(self.slot_pos, "cache.slot_pos", (b, hkv, Bc), torch.int32, dev)
        _need(self.slot_prio, "cache.slot_prio", (b, hkv, Bc), torch.float32, dev)
        _need(self.ring, "cache.ring", (b, hkv, window), torch.int32, dev)
        if self.state is not None:
            _need(self.state, "cache.state", (b, hkv, CACHE_STATE_WORDS), torch.int32, dev)


def new_decode_cache(batch: int, n_kv_heads: int, head_dim: int, sink: int, window: int,
                     topk: int, dtype: torch.dtype = torch.bfloat16, device="cuda") -> DecodeCache:
    Bc = sink + window + topk
    z = dict(device=device)
    return DecodeCache(
        torch.zeros((batch, n_kv_heads, Bc, head_dim), dtype=dtype, **z),
        torch.zeros((batch, n_kv_heads, Bc, head_dim), dtype=dtype, **z),
        torch.full((batch, n_kv_heads, Bc), -1, dtype=torch.int32, **z),
        torch.zeros((batch, n_kv_heads, Bc), dtype=torch.float32, **z),
        torch.zeros((batch, n_kv_heads, max(window, 1)), dtype=torch.int32, **z),
        torch.zeros((batch, n_kv_heads, CACHE_STATE_WORDS), dtype=torch.int32, **z))


def decode_step(cache: DecodeCache, pos: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                v_new: torch.Tensor, prio_leaving: torch.Tensor, sink: int, window: int, topk: int,
                softmax_scale: float = 0.0, out_dtype: torch.dtype = torch.float32,
                o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None):
    """One decode step for every sequence; updates `cache` in place; returns (o, lse)."""
    b, hq, D = q.shape
    hkv = k_new.shape[1]
    dev = q.device
    Bc = sink + window + topk
    _need(q, "q", (b, hq, D), q.dtype)
    _need(k_new, "k_new", (b, hkv, D), q.dtype, dev)
    _need(v_new, "v_new", (b, hkv, D), q.dtype, dev)
    _need(prio_leaving, "prio_leaving", (b, hkv), torch.float32, dev)
    _need(pos, "pos", (b,), torch.int32, dev)
    cache.check(b, hkv, Bc, D, window, q.dtype, dev)
    o = torch.empty((b, hq, D), dtype=out_dtype, device=dev) if o is None else o
    lse = torch.empty((b, hq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (b, hq, D), out_dtype, dev)
    _need(lse, "lse", (b, hq), torch.float32, dev)
    pr = Problem(b, hq, hkv, 0, D, sink, window, topk, softmax_scale, _dtype_code(q.dtype),
                 _dtype_code(out_dtype))
    n = workspace_size(CALL_DECODE, pr)
    if ws is None:
        ws, n = _workspace(CALL_DECODE, pr, dev)
    elif ws.numel() < n or ws.data_ptr() % 256:
        raise KvpopError("decode workspace too small or not 256-byte aligned")
    cc = cache.c()
    c = pr.c()
    _status(lib().kvpop_decode_step(ctypes.byref(c), ctypes.byref(cc), _vp(pos), _vp(q),
                                    _vp(k_new), _vp(v_new), _vp(prio_leaving), _vp(o), _vp(lse),
                                    _vp(ws), n, _stream(dev)), "kvpop_decode_step")
    return o, lse


def decode_step_noalloc(cache: DecodeCache, pos: torch.Tensor, q: torch.Tensor,
                        k_new: torch.Tensor, v_new: torch.Tensor, prio_leaving: torch.Tensor,
                        sink: int, window: int, topk: int, softmax_scale: float = 0.0,
                        out_dtype: torch.dtype = torch.float32,
                        o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """decode_step through kvpop_decode_step_noalloc: the library's fixed device
    scratch instead of a workspace (no allocation inside the call; pass `o`
    and `lse` to allocate nothing here either)."""
    b, hq, D = q.shape
    hkv = k_new.shape[1]
    dev = q.device
    Bc = sink + window + topk
    _need(q, "q", (b, hq, D), q.dtype)
    _need(k_new, "k_new", (b, hkv, D), q.dtype, dev)
    _need(v_new, "v_new", (b, hkv, D), q.dtype, dev)
    _need(prio_leaving, "prio_leaving", (b, hkv), torch.float32, dev)
    _need(pos, "pos", (b,), torch.int32, dev)
    cache.check(b, hkv, Bc, D, window, q.dtype, dev)
    o = torch.empty((b, hq, D), dtype=out_dtype, device=dev) if o is None else o
    lse = torch.empty((b, hq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (b, hq, D), out_dtype, dev)
    _need(lse, "lse", (b, hq), torch.float32, dev)
    pr = Problem(b, hq, hkv, 0, D, sink, window, topk, softmax_scale, _dtype_code(q.dtype),
                 _dtype_code(out_dtype))
    cc = cache.c()
    c = pr.c()
    _status(lib().kvpop_decode_step_noalloc(ctypes.byref(c), ctypes.byref(cc), _vp(pos), _vp(q),
                                            _vp(k_new), _vp(v_new), _vp(prio_leaving), _vp(o),
                                            _vp(lse), _stream(dev)), "kvpop_decode_step_noalloc")
    return o, lse


def cache_from_prefill(cache: DecodeCache, k: torch.Tensor, v: torch.Tensor, prio: torch.Tensor,
                       rank: torch.Tensor, tau: torch.Tensor, sink: int, window: int,
                       topk: int) -> DecodeCache:
    """Fill `cache` with the kept set of the prompt's last row (see
    kvpop_cache_from_prefill); decoding then continues at p = S."""
    b, hkv, S, D = k.shape
    dev = k.device
    Bc = sink + window + topk
    _need(k, "k", (b, hkv, S, D), k.dtype, dev)
    _need(v, "v", (b, hkv, S, D), k.dtype, dev)
    _need(prio, "prio", (b, hkv, S), torch.float32, dev)
    _need(rank, "rank", (b, hkv, S), torch.int32, dev)
    _need(tau, "tau", (b, hkv, S), torch.int32, dev)
    cache.check(b, hkv, Bc, D, window, k.dtype, dev)
    pr = Problem(b, hkv, hkv, S, D, sink, window, topk, 0.0, _dtype_code(k.dtype), 0)
    c, cc = pr.c(), cache.c()
    _status(lib().kvpop_cache_from_prefill(ctypes.byref(c), ctypes.byref(cc), _vp(k), _vp(v),
                                           _vp(prio), _vp(rank), _vp(tau), _stream(dev)),
            "kvpop_cache_from_prefill")
    return cache


def target_score(target: torch.Tensor, n_kv_heads: int, window: int, eps: float,
                 score: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Aggregated target score [b, Hkv, S] from the per-query-head future
    target [b, Hq, S] (see kvpop_target_score)."""
    b, hq, S = target.shape
    dev = target.device
    _need(target, "target", (b, hq, S), torch.float32, dev)
    score = torch.empty((b, n_kv_heads, S), dtype=torch.float32, device=dev) if score is None else score
    _need(score, "score", (b, n_kv_heads, S), torch.float32, dev)
    pr = Problem(b, hq, n_kv_heads, S, 128, 0, window, 0, 0.0, 0, 0)
    c = pr.c()
    _status(lib().kvpop_target_score(ctypes.byref(c), _vp(target), float(eps), _vp(score),
                                     _stream(dev)), "kvpop_target_score")
    return score


def boundary_labels(score: torch.Tensor, log_gamma: torch.Tensor, decay_step: int, sink: int,
                    window: int, topk: int, t_bnd: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None):
    """t_bnd, y = boundary_labels(score[b, Hkv, S], log_gamma[Hkv], n, s, w, k):
    the teacher's boundary token and label of every query row (see
    kvpop_boundary_labels)."""
    b, hkv, S = score.shape
    dev = score.device
    _need(score, "score", (b, hkv, S), torch.float32)
    _need(log_gamma, "log_gamma", (hkv,), torch.float32, dev)
    t_bnd = torch.empty((b, hkv, S), dtype=torch.int32, device=dev) if t_bnd is None else t_bnd
    y = torch.empty((b, hkv, S), dtype=torch.int32, device=dev) if y is None else y
    _need(t_bnd, "t_bnd", (b, hkv, S), torch.int32, dev)
    _need(y, "y", (b, hkv, S), torch.int32, dev)
    pr = Problem(b, hkv, hkv, S, 128, sink, window, topk, 0.0, 0, 0)
    c = pr.c()
    _status(lib().kvpop_boundary_labels(ctypes.byref(c), _vp(score), _vp(log_gamma),
                                        int(decay_step), _vp(t_bnd), _vp(y), _stream(dev)),
            "kvpop_boundary_labels")
    return t_bnd, y


def masked_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, rank: torch.Tensor, tau: torch.Tensor, dout: torch.Tensor,
                    sink: int, window: int, topk: int, softmax_scale: float = 0.0,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None):
    """dq, dk, dv = masked_attn_bwd(q, k, v, o, lse, rank, tau, dout, s, w, k): the
    gradients of masked_attn_fwd for the upstream gradient dout of o (see
    kvpop_masked_attn_bwd); q, k, v, dout bfloat16, o and lse the forward's."""
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    dev = q.device
    bf = torch.bfloat16
    _need(q, "q", (b, hq, S, D), bf)
    _need(k, "k", (b, hkv, S, D), bf, dev)
    _need(v, "v", (b, hkv, S, D), bf, dev)
    _need(dout, "dout", (b, hq, S, D), bf, dev)
    _need(o, "o", (b, hq, S, D), o.dtype, dev)
    _need(lse, "lse", (b, hq, S), torch.float32, dev)
    _need(rank, "rank", (b, hkv, S), torch.int32, dev)
    _need(tau, "tau", (b, hkv, S), torch.int32, dev)
    f32 = torch.float32
    dq = torch.empty((b, hq, S, D), dtype=f32, device=dev) if dq is None else dq
    dk = torch.empty((b, hkv, S, D), dtype=f32, device=dev) if dk is None else dk
    dv = torch.empty((b, hkv, S, D), dtype=f32, device=dev) if dv is None else dv
    _need(dq, "dq", (b, hq, S, D), f32, dev)
    _need(dk, "dk", (b, hkv, S, D), f32, dev)
    _need(dv, "dv", (b, hkv, S, D), f32, dev)
    pr = Problem(b, hq, hkv, S, D, sink, window, topk, softmax_scale, _dtype_code(bf),
                 _dtype_code(o.dtype))
    ws, n = _workspace(CALL_MASKED_BWD, pr, dev)
    c = pr.c()
    _status(lib().kvpop_masked_attn_bwd(ctypes.byref(c), _vp(q), _vp(k), _vp(v), _vp(o), _vp(lse),
                                        _vp(rank), _vp(tau), _vp(dout), _vp(dq), _vp(dk), _vp(dv),
                                        _vp(ws), n, _stream(dev)), "kvpop_masked_attn_bwd")
    return dq, dk, dv
