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

# Gradients of the masked attention: P and dS enter the MFMA products rounded
# to bfloat16 (relative error 2^-9 per term) and every sum is float32, so each
# gradient tensor is held to 1e-2 relative in the Frobenius norm and 2e-2 of
# its largest entry per element; one wrongly masked key moves an element by
# O(its size).
BWD_TOL = {"fro": 1e-2, "max": 2e-2}
