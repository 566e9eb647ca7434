"""kvpop_decode_step_noalloc (the decode step with the library's fixed device
scratch instead of a workspace, for callers that cannot allocate) against
kvpop_decode_step through the C ABI: two decode runs in a row, the second on a
smaller problem, each step's o and lse and the final cache equal bit for bit.
Both runs split the cache over several workgroups, so the scratch is used."""
import pytest
import torch

import fixed_budget_sparse_amd as kv
from gpu_util import announce, device

pytestmark = pytest.mark.gpu

RUNS = [
    # nseq, Hq, Hkv, D, s, w, k, steps, cache dtype, out dtype
    (8, 32, 8, 128, 4, 32, 476, 600, torch.bfloat16, torch.bfloat16),   # 4 splits
    (2, 8, 2, 64, 2, 8, 200, 260, torch.float32, torch.float32),        # 2 splits, smaller
]


def _run(nseq, hq, hkv, D, s, w, k, steps, cdt, odt, seed):
    dev = device()
    Bc = s + w + k
    pr = kv.Problem(nseq, hq, hkv, 0, D, s, w, k, 0.0, 0 if cdt == torch.bfloat16 else 1, 0)
    assert kv.workspace_size(3, pr) > 0                      # several splits: scratch in use
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    ca = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=cdt, device=dev)
    cb = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=cdt, device=dev)
    ob = torch.empty((nseq, hq, D), dtype=odt, device=dev)
    lb = torch.empty((nseq, hq), dtype=torch.float32, device=dev)
    mismatch = torch.zeros((), dtype=torch.int32, device=dev)
    for p in range(steps):
        q = torch.randn((nseq, hq, D), generator=g, device=dev).to(cdt)
        kn = torch.randn((nseq, hkv, D), generator=g, device=dev).to(cdt)
        vn = torch.randn((nseq, hkv, D), generator=g, device=dev).to(cdt)
        pl = torch.randn((nseq, hkv), generator=g, device=dev)
        pos = torch.full((nseq,), p, dtype=torch.int32, device=dev)
        oa, la = kv.decode_step(ca, pos, q, kn, vn, pl, s, w, k, out_dtype=odt)
        kv.decode_step_noalloc(cb, pos, q, kn, vn, pl, s, w, k, out_dtype=odt, o=ob, lse=lb)
        mismatch += (~torch.eq(oa, ob)).sum() + (~torch.eq(la, lb)).sum()
    torch.cuda.synchronize()
    assert int(mismatch) == 0
    for name in ("k", "v", "slot_pos", "slot_prio", "ring", "state"):
        assert torch.equal(getattr(ca, name), getattr(cb, name)), name
    # the cache filled and then evicted: every slot holds a token
    assert int((ca.slot_pos >= 0).sum()) == nseq * hkv * min(steps, Bc)


def test_decode_noalloc_matches_decode_step():
    for i, run in enumerate(RUNS):
        announce(f"decode_step_noalloc run {i}: {run[:8]}")
        _run(*run, seed=900 + i)
