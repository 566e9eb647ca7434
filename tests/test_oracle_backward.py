"""Pins of the oracle's masked attention backward ([Notes] §2.3: the student's
sparse forward over the kept set): central finite differences of the forward,
an independent autograd derivation of dense causal attention (k >= S keeps
every causal key), and identities of the softmax Jacobian."""
import numpy as np
import pytest
import torch

import oracle as orc


def _case(seed, b=1, hq=2, hkv=1, S=14, D=4, s=2, w=3, k=3, ties=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, hq, S, D))
    kk = rng.standard_normal((b, hkv, S, D))
    v = rng.standard_normal((b, hkv, S, D))
    prio = rng.standard_normal((b, hkv, S))
    if ties:
        prio = np.round(prio)
    rank = orc.priority_ranks(prio)
    tau = orc.thresholds_by_selection(rank, s, w, k)
    dout = rng.standard_normal((b, hq, S, D))
    return q, kk, v, rank, tau, dout


@pytest.mark.parametrize("seed,kw", [(1, {}), (2, dict(hq=4, hkv=2, S=16, k=4)),
                                     (3, dict(s=0, w=1, k=2, ties=True)), (4, dict(k=0, w=2))])
def test_finite_differences(seed, kw):
    q, kk, v, rank, tau, dout = _case(seed, **kw)
    s, w = kw.get("s", 2), kw.get("w", 3)
    dQ, dK, dV = orc.masked_attention_backward(q, kk, v, rank, tau, s, w, dout)

    def loss(q_, k_, v_):
        O, _ = orc.masked_attention(q_, k_, v_, rank, tau, s, w)
        return float((O * dout).sum())

    h = 1e-6
    for grad, which in ((dQ, 0), (dK, 1), (dV, 2)):
        base = [q, kk, v]
        x = base[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p, args_m = list(base), list(base)
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-6 * max(1.0, np.abs(grad).max()), which


def test_dense_causal_matches_autograd():
    # k >= S keeps every causal key: the gradients are those of dense causal
    # attention, here differentiated by torch autograd from its own forward.
    b, hq, hkv, S, D = 1, 4, 2, 24, 8
    q, kk, v, rank, tau, dout = _case(5, b, hq, hkv, S, D, s=1, w=4, k=S)
    dQ, dK, dV = orc.masked_attention_backward(q, kk, v, rank, tau, 1, 4, dout)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, kk, v))
    G = hq // hkv
    K = tk.repeat_interleave(G, dim=1)
    V = tv.repeat_interleave(G, dim=1)
    z = (tq @ K.transpose(-1, -2)) / np.sqrt(D)
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    z = z.masked_fill(~causal, float("-inf"))
    O = torch.softmax(z, dim=-1) @ V
    (O * torch.tensor(dout)).sum().backward()
    assert np.allclose(tq.grad.numpy(), dQ, atol=1e-10)
    assert np.allclose(tk.grad.numpy(), dK, atol=1e-10)
    assert np.allclose(tv.grad.numpy(), dV, atol=1e-10)


def test_softmax_jacobian_identities():
    q, kk, v, rank, tau, dout = _case(6, hq=2, hkv=1, S=30, D=6, s=3, w=4, k=5)
    dQ, dK, dV = orc.masked_attention_backward(q, kk, v, rank, tau, 3, 4, dout)
    # each row's probabilities sum to one, so the value gradients sum to the
    # upstream gradient over the group's rows
    assert np.allclose(dV.sum(axis=2)[0, 0], dout[0].sum(axis=(0, 1)), atol=1e-10)
    # equal keys: the logits of a row shift together and dQ vanishes
    k_eq = np.repeat(kk[:, :, :1], kk.shape[2], axis=2)
    dQ2, _, _ = orc.masked_attention_backward(q, k_eq, v, rank, tau, 3, 4, dout)
    assert np.abs(dQ2).max() <= 1e-12
