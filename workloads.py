"""Seeded synthetic workloads for the KVpop fixed-budget KV-cache hot path.

This module only draws inputs: it holds none of the method's arithmetic, so both
the CPU oracle (``oracle/``) and the HIP library's callers (tests, bench, smoke)
can take their inputs from here without sharing any computation.

Input recipe (the same for every configuration):
  * Q, K, V ~ N(0, 1) drawn in float32; keys 0..3 of every (batch, kv-head) are
    multiplied by 4 (a sink-like mass on the first keys).  For bfloat16
    configurations the draws are rounded to nearest-even bfloat16 and held as
    exactly representable float32 values, so host and device see the same bits.
  * Per-token priorities ~ N(0, 1) float32, one per (batch, kv-head, token).
  * Decode steps draw q, k_new, v_new ~ N(0, 1) (rounded like Q/K/V) and a
    priority table prio_table[b, h, t] ~ N(0, 1) for the token leaving the window.
  * Upstream gradients dO of the attention output ~ N(0, 1), rounded like Q.
  * Teacher-label inputs: stand-in target scores r_t ~ N(-9.5, 1.5) float32 per
    (batch, kv-head, token) (the log of a future attention mass averaged over
    ~10^4 queries sits near there), per-head log(gamma_h) ~ U(-0.03, -0.003)
    and a decay step of 64 tokens (the pages give no values for n or gamma).
    With these the decay over a 16k context (up to 256 steps) is comparable to
    the spread of the scores, so the newcomer is kept in roughly 35-60 % of
    the rows of a head rather than always (a stronger decay makes the newest
    token win every comparison).

These stand in for Qwen3-4B/8B attention activations at the sequence lengths
the KVpop paper trains and evaluates at (arXiv 2607.05061, section 4); no
dataset or trained weights are used.

Seeding: every tensor has its own stream
``np.random.default_rng([seed, config_id, tensor_id])`` so that any tensor can be
regenerated independently of the others.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and budget of one synthetic workload (one attention layer)."""

    name: str
    config_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    dtype: str            # "f32" or "bf16"
    sink: int
    window: int
    topk: int
    seed: int = 0

    @property
    def budget(self) -> int:
        """B = s + w + k, the per-KV-head cache size."""
        return self.sink + self.window + self.topk

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# The five workloads, in order (ids 0..4): tiny reference, 16k and 32k layers, decode, long context.
TINY = Workload("tiny-f32-S512", 0, 1, 2, 1, 64, 512, "f32", 4, 32, 64)
QWEN3_4B_S16K = Workload("qwen3-4b-layer-S16384-B2048", 1, 1, 32, 8, 128, 16384, "bf16",
                         16, 512, 1520)
QWEN3_8B_S32K = Workload("qwen3-8b-layer-S32768-B4096", 2, 1, 32, 8, 128, 32768, "bf16",
                         16, 1024, 3056)
# Decode: 64 sequences, cache of B = 2048 per KV head; seq_len is the number of
# positions the prio table covers (warm-up 0..4095, timed 4096..5119).
DECODE_B2048 = Workload("decode-64seq-B2048", 3, 64, 32, 8, 128, 5120, "bf16", 16, 512, 1520)
LONG_S128K = Workload("long-S131072-B4096", 4, 1, 32, 8, 128, 131072, "bf16", 16, 1024, 3056)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, QWEN3_4B_S16K, QWEN3_8B_S32K, DECODE_B2048, LONG_S128K)}

# tensor ids for the per-tensor seed streams
_TID = {"q": 0, "k": 1, "v": 2, "prio": 3, "dec_q": 4, "dec_k": 5, "dec_v": 6,
        "dec_prio": 7, "label_score": 8, "label_gamma": 9, "dout": 10}

LABEL_DECAY_STEP = 64


def rng_for(seed: int, config_id: int, tensor: str, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, config_id, _TID[tensor], extra])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Finite inputs only (the draws here are Gaussian)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def make_prefill(wl: Workload, seq_len: int | None = None, batch: int | None = None,
                 seed: int | None = None, sink_scale_keys: int = 4):
    """Return dict(q, k, v, prio) as float32 numpy arrays (bf16-exact if bf16).

    Shapes: q [b, Hq, S, D], k/v [b, Hkv, S, D], prio [b, Hkv, S].
    ``seq_len``/``batch`` override the workload's sizes (for reduced parity cases).
    """
    S = wl.seq_len if seq_len is None else seq_len
    b = wl.batch if batch is None else batch
    sd = wl.seed if seed is None else seed
    q = _normal(rng_for(sd, wl.config_id, "q"), (b, wl.n_q_heads, S, wl.head_dim), wl.dtype)
    k = rng_for(sd, wl.config_id, "k").standard_normal(
        size=(b, wl.n_kv_heads, S, wl.head_dim), dtype=np.float32)
    k[:, :, :sink_scale_keys, :] *= 4.0
    if wl.dtype == "bf16":
        k = round_to_bf16(k)
    v = _normal(rng_for(sd, wl.config_id, "v"), (b, wl.n_kv_heads, S, wl.head_dim), wl.dtype)
    prio = rng_for(sd, wl.config_id, "prio").standard_normal(
        size=(b, wl.n_kv_heads, S), dtype=np.float32)
    return {"q": q, "k": k, "v": v, "prio": prio}


def make_decode_step(wl: Workload, step: int, batch: int | None = None, seed: int | None = None):
    """Inputs of decode step ``step`` (the same step index for every sequence).

    Returns dict(q [b, Hq, D], k_new [b, Hkv, D], v_new [b, Hkv, D]) float32
    (bf16-exact if bf16)."""
    b = wl.batch if batch is None else batch
    sd = wl.seed if seed is None else seed
    D = wl.head_dim
    q = _normal(rng_for(sd, wl.config_id, "dec_q", step), (b, wl.n_q_heads, D), wl.dtype)
    kn = rng_for(sd, wl.config_id, "dec_k", step).standard_normal(
        size=(b, wl.n_kv_heads, D), dtype=np.float32)
    if step < 4:
        kn *= 4.0
    if wl.dtype == "bf16":
        kn = round_to_bf16(kn)
    vn = _normal(rng_for(sd, wl.config_id, "dec_v", step), (b, wl.n_kv_heads, D), wl.dtype)
    return {"q": q, "k_new": kn, "v_new": vn}


def make_decode_prio_table(wl: Workload, n_tokens: int | None = None, batch: int | None = None,
                           seed: int | None = None) -> np.ndarray:
    """prio_table[b, h, t] ~ N(0,1): the priority token t receives when it leaves
    the window (read at step t + w)."""
    b = wl.batch if batch is None else batch
    T = wl.seq_len if n_tokens is None else n_tokens
    sd = wl.seed if seed is None else seed
    return rng_for(sd, wl.config_id, "dec_prio").standard_normal(
        size=(b, wl.n_kv_heads, T), dtype=np.float32)


def make_label_inputs(wl: Workload, seq_len: int | None = None, batch: int | None = None,
                      seed: int | None = None):
    """Teacher-label inputs: score [b, Hkv, S] float32 (stand-in target scores)
    and log_gamma [Hkv] float32."""
    b = wl.batch if batch is None else batch
    S = wl.seq_len if seq_len is None else seq_len
    sd = wl.seed if seed is None else seed
    score = (rng_for(sd, wl.config_id, "label_score").standard_normal(
        size=(b, wl.n_kv_heads, S), dtype=np.float32) * np.float32(1.5) - np.float32(9.5))
    log_gamma = rng_for(sd, wl.config_id, "label_gamma").uniform(
        -0.03, -0.003, size=wl.n_kv_heads).astype(np.float32)
    return {"score": score.astype(np.float32), "log_gamma": log_gamma}


def scaled(wl: Workload, **over) -> Workload:
    """A copy of ``wl`` with some fields replaced (reduced parity cases)."""
    return dataclasses.replace(wl, **over)


# --------------------------------------------------------------------------
# Device-side draws for the full-size cases.  The same recipe (N(0,1), keys
# 0..3 x4, bfloat16 rounding to nearest even, N(0,1) priorities) drawn with
# torch's seeded generator directly in device memory, so that inputs of
# hundreds of millions of elements need not pass through the host.  Host
# copies of whatever a check needs are taken from these tensors.
# --------------------------------------------------------------------------
def torch_seed(seed: int, config_id: int, tensor: str, extra: int = 0) -> int:
    """A 63-bit seed for torch.Generator, one per (seed, config, tensor, extra)."""
    st = np.random.SeedSequence([seed, config_id, _TID[tensor], extra]).generate_state(2)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _device_normal(shape, seed: int, device, dtype: str, scale_first: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale_first:
        x[..., :scale_first, :] *= 4.0
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def make_prefill_device(wl: Workload, device, seq_len: int | None = None,
                        batch: int | None = None, seed: int | None = None,
                        sink_scale_keys: int = 4):
    """dict(q, k, v, prio) as device tensors: q [b, Hq, S, D], k/v [b, Hkv, S, D]
    in bfloat16 (float32 for float32 workloads), prio [b, Hkv, S] float32."""
    S = wl.seq_len if seq_len is None else seq_len
    b = wl.batch if batch is None else batch
    sd = wl.seed if seed is None else seed
    c = wl.config_id
    D = wl.head_dim
    q = _device_normal((b, wl.n_q_heads, S, D), torch_seed(sd, c, "q"), device, wl.dtype)
    k = _device_normal((b, wl.n_kv_heads, S, D), torch_seed(sd, c, "k"), device, wl.dtype,
                       sink_scale_keys)
    v = _device_normal((b, wl.n_kv_heads, S, D), torch_seed(sd, c, "v"), device, wl.dtype)
    prio = _device_normal((b, wl.n_kv_heads, S, 1), torch_seed(sd, c, "prio"), device, "f32")
    return {"q": q, "k": k, "v": v, "prio": prio[..., 0].contiguous()}


def make_grad_device(wl: Workload, device, seq_len: int | None = None, seed: int | None = None):
    """Upstream gradient dO ~ N(0, 1) of the attention output, [b, Hq, S, D],
    rounded like Q (bfloat16 for bfloat16 workloads), on the device."""
    S = wl.seq_len if seq_len is None else seq_len
    sd = wl.seed if seed is None else seed
    return _device_normal((wl.batch, wl.n_q_heads, S, wl.head_dim),
                          torch_seed(sd, wl.config_id, "dout"), device, wl.dtype)


def make_decode_stream_device(wl: Workload, device, n_steps: int, batch: int | None = None,
                              seed: int | None = None):
    """Per-step decode inputs for steps 0..n_steps-1 as device tensors:
    k_new/v_new [n_steps, b, Hkv, D] (token p's K/V at index p; tokens 0..3 x4)
    and prio_table [b, Hkv, n_steps] float32 (read at step t + w)."""
    b = wl.batch if batch is None else batch
    sd = wl.seed if seed is None else seed
    c = wl.config_id
    D = wl.head_dim
    shape = (b, wl.n_kv_heads, n_steps, D)
    k = _device_normal(shape, torch_seed(sd, c, "dec_k"), device, wl.dtype, 4)
    v = _device_normal(shape, torch_seed(sd, c, "dec_v"), device, wl.dtype)
    prio = _device_normal((b, wl.n_kv_heads, n_steps, 1), torch_seed(sd, c, "dec_prio"),
                          device, "f32")
    return {"k_new": k.permute(2, 0, 1, 3).contiguous(),
            "v_new": v.permute(2, 0, 1, 3).contiguous(),
            "prio_table": prio[..., 0].contiguous()}


def make_decode_query_device(wl: Workload, device, step: int, batch: int | None = None,
                             seed: int | None = None):
    """The query of decode step ``step``: [b, Hq, D] on the device."""
    b = wl.batch if batch is None else batch
    sd = wl.seed if seed is None else seed
    return _device_normal((b, wl.n_q_heads, wl.head_dim), torch_seed(sd, wl.config_id, "dec_q",
                                                                     step), device, wl.dtype)
