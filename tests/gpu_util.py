"""Helpers shared by the GPU tests (comparison metrics, device setup).

Metrics (the tolerance readings of the design notes):
  S, dW: per-row normwise relative error, max_i max_j |x_ij - y_ij| / max_j |y_ij|
  v:     elementwise relative error (v > 0)
  sqnorm: scalar relative error
  bf16 W: |W_gpu - W_ref| <= 1 bf16 ulp of W_ref, elementwise
"""
import numpy as np
import pytest
import torch

BF16_TOL = 2e-2   # bf16 inputs, fp32 accumulation
F32_TOL = 1e-5    # fp32 path


def device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)


def rownorm_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float((np.abs(got - ref) / np.abs(ref)).max())


def bf16_ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, 2.0 ** (e - 7), 2.0 ** -133)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
