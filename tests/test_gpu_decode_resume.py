"""A decode run checkpointed to host memory and resumed in a fresh cache is
bit-identical to the uninterrupted run.

The cache arrays (K, V, slot positions and priorities, the window ring and the
next step's record) are the whole decode state: the library keeps nothing
between calls.  So copying them
to the host at some position, restoring them into newly allocated device
arrays and continuing must reproduce every later output and the final cache
bit for bit, including across the fill (p < B) to steady-state boundary and
the window boundary where tokens start to compete for the long-range slots."""
import pytest
import torch

import fixed_budget_sparse_amd as kv
from gpu_util import announce, device

pytestmark = pytest.mark.gpu


def _cache_arrays(c):
    return c.arrays()


@pytest.mark.parametrize("cut", [37, 150, 301])
def test_decode_checkpoint_resume_bit_identical(cut):
    announce(f"decode checkpoint at step {cut} and resume in a fresh cache")
    dev = device()
    nseq, hq, hkv, D, s, w, k = 3, 8, 2, 128, 4, 32, 100     # B = 136
    n_steps = 400
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    qs = torch.randn((n_steps, nseq, hq, D), generator=g, device=dev).to(bf)
    kn = torch.randn((n_steps, nseq, hkv, D), generator=g, device=dev).to(bf)
    vn = torch.randn((n_steps, nseq, hkv, D), generator=g, device=dev).to(bf)
    pr = torch.randn((n_steps, nseq, hkv), generator=g, device=dev)
    pos = torch.arange(n_steps, dtype=torch.int32, device=dev)[:, None].repeat(1, nseq).contiguous()

    def run(cache, lo, hi, outs):
        for p in range(lo, hi):
            o, lse = kv.decode_step(cache, pos[p], qs[p], kn[p], vn[p], pr[p], s, w, k,
                                    out_dtype=torch.float32)
            outs.append((o, lse))

    full = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=bf, device=dev)
    ref = []
    run(full, 0, n_steps, ref)

    first = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=bf, device=dev)
    got = []
    run(first, 0, cut, got)
    torch.cuda.synchronize()
    saved = [t.cpu() for t in _cache_arrays(first)]          # the checkpoint
    del first
    resumed = kv.new_decode_cache(nseq, hkv, D, s, w, k, dtype=bf, device=dev)
    for dst, src in zip(_cache_arrays(resumed), saved):
        dst.copy_(src.to(dev))
    run(resumed, cut, n_steps, got)
    torch.cuda.synchronize()

    for p, ((o0, l0), (o1, l1)) in enumerate(zip(ref, got)):
        assert torch.equal(o0.view(torch.int32), o1.view(torch.int32)), p
        assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), p
    for a, b in zip(_cache_arrays(full), _cache_arrays(resumed)):
        if a.is_floating_point():
            a, b = a.view(torch.int16 if a.element_size() == 2 else torch.int32), \
                b.view(torch.int16 if b.element_size() == 2 else torch.int32)
        assert torch.equal(a, b)
