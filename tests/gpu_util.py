"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


def tdtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def announce(msg: str):
    print(f"[case] {msg}", flush=True)


# tolerances (bf16 inputs: O <= 1e-2 max-abs, LSE <= 1e-3, targets <= 5e-3 where > -20;
# float32 inputs: float32 accumulation only, so much tighter)
TOL = {"bf16": {"o": 1e-2, "lse": 1e-3, "tgt": 5e-3},
       "f32": {"o": 1e-4, "lse": 1e-4, "tgt": 1e-4}}

# Gradients of the masked attention.  P enters the dV product and dS the dQ
# and dK products rounded to bfloat16 (round to nearest even: relative error
# below 2^-9, RMS 2^-9/sqrt(3) ~ 1.1e-3 per term, unbiased), every sum is
# float32.  A gradient is a sum of many such terms of mixed sign, so its
# error relative to its Frobenius norm is about that RMS (1.4-1.9e-3
# measured); the largest element error relative to the largest element is a
# little higher where rows are short (up to 2.9e-3).  With a bfloat16 forward
# output, D_i = <dO_i, O_i> also carries O's rounding, and dP - D cancels, so
# dQ and dK move up to 4.4e-3 (Frobenius) and 5.4e-3 (largest element).  The
# bars sit about 1.4-1.8x above the worst measured case of each kind, keyed
# by the forward output's dtype; a wrongly masked key shifts the affected
# rows by its whole probability.
BWD_TOL = {"f32": {"fro": 3e-3, "max": 4e-3},
           "bf16": {"fro": 6e-3, "max": 8e-3}}
