"""Python binding of libkvpop (KVpop fixed-budget sparse KV cache, MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvpop.so``.  PyTorch provides device memory and the current HIP stream.
If the library is missing or the GPU is not available the calls raise; there
is no CPU fallback.
"""
from __future__ import annotations

from .binding import (  # noqa: F401
    KvpopError,
    Problem,
    DecodeCache,
    lib,
    library_path,
    abi_version,
    debug_reverse_launch_order,
    workspace_size,
    thresholds,
    masked_attn_fwd,
    future_target,
    decode_step,
    decode_step_noalloc,
    new_decode_cache,
    cache_from_prefill,
    target_score,
    boundary_labels,
    masked_attn_bwd,
    EXPORTED_SYMBOLS,
)
