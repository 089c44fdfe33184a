"""Helpers shared by the GPU tests (comparison metrics, device setup).

Metrics (the tolerance readings of the design notes):
  S, dW: per-row normwise relative error, max_i max_j |x_ij - y_ij| / max_j |y_ij|
         (for a stored fp32 W, after one fp32 ulp of the result: w_update_err)
  v:     elementwise relative error (v > 0)
  sqnorm: scalar relative error
  bf16 W: |W_gpu - W_ref| <= sum over the steps so far of (1 bf16 ulp of
          that step's W_ref + 2e-2 * max_j |that step's dW_ref,ij|),
          elementwise: one rounding of the stored value plus the tolerance
          of the update itself, per step, since each side rounds on its own
          path and starts the next step from its own stored W
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


def f32_ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, 2.0 ** (e - 23), 2.0 ** -149)


def w_update_err(W_gpu, W_ref, W_old):
    """Per-row normwise error of an fp32 W update, after allowing the one
    fp32 rounding of the stored result: max_j (|W_gpu - W_ref| - ulp(W_ref))+
    over max_j |W_ref - W_old|."""
    W_gpu = np.asarray(W_gpu, dtype=np.float64)
    W_ref = np.asarray(W_ref, dtype=np.float64)
    W_old = np.asarray(W_old, dtype=np.float64)
    if W_gpu.size == 0:
        return 0.0
    num = np.maximum(np.abs(W_gpu - W_ref) - f32_ulp(W_ref), 0.0).max(axis=1)
    den = np.abs(W_ref - W_old).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def bf16_w_check(W_gpu, W_ref, W_old, tol=BF16_TOL, prior=None):
    """Return (ok, worst ratio, allowance) for a bf16 W update against the
    fp64 oracle. Each side rounds W to bf16 on its own path, so one step
    allows one ulp of the stored result plus the update's own tolerance
    (tol x the row's largest oracle update). When state is carried over
    several steps, each side starts the next step from its own stored W, so
    the difference carried in is added: pass the previous step's allowance
    as `prior` (elementwise), and this step's comes back as the third value."""
    W_gpu = np.asarray(W_gpu, dtype=np.float64)
    W_ref = np.asarray(W_ref, dtype=np.float64)
    W_old = np.asarray(W_old, dtype=np.float64)
    W_ref_b = torch.from_numpy(W_ref).to(torch.bfloat16).double().numpy()
    upd = np.abs(W_ref - W_old).max(axis=1, keepdims=True)
    allowed = bf16_ulp(W_ref_b) + tol * upd
    if prior is not None:
        allowed = allowed + prior
    ratio = np.abs(W_gpu - W_ref_b) / allowed
    return bool(np.all(ratio <= 1.0)), float(ratio.max()) if ratio.size else 0.0, allowed


def f32(x) -> float:
    """A hyper-parameter as the C ABI receives it (a C float): the oracle is
    given the same value the kernels compute with."""
    return float(np.float32(x))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
