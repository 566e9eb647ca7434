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
# at most 2^-8, RMS about 1.7e-3 per term, unbiased), every sum is float32;
# the forward's PV product takes its probabilities rounded the same way
# (relative to a lazily moved reference maximum, so even a row's largest
# probability is rounded), and D_i = <dO_i, O_i> carries that rounding of O.
# Over the whole tensor the errors of many mixed-sign terms average out: the
# error relative to the Frobenius norm measures 1.4-1.9e-3 with a float32 O
# and up to 4.4e-3 with a bfloat16 O (whose own rounding adds to D); the
# Frobenius bars sit about 1.4x above the worst measured case.  Element by
# element, a row that one key dominates has dP - D cancel, so D's error
# reaches dS of that key undiminished; the reduced cases bound every element
# by the first-order sum of these roundings, and the full-size case, which
# the oracle cannot bound element by element in seconds, keeps a largest-
# element bar (bf16 O: 8e-3 of the largest element).  A wrongly masked key
# shifts the affected rows by its whole probability.
BWD_TOL = {"f32": {"fro": 3e-3},
           "bf16": {"fro": 6e-3, "max": 8e-3}}
BF16_U = 2.0 ** -8      # unit roundoff of bfloat16, round to nearest even
