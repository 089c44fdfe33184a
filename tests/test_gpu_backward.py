"""GPU parity of the backward input gradient dX = dY W and of the launch that
computes it beside the sketch's fold (logra_backward_dx,
logra_backward_dx_sketch), through the C ABI against the oracle: dX per row
normwise at 2e-2 (bf16 inputs and output, fp32 accumulation), S as in the
sketch tests, dX of the fused launch bit-identical to the product alone, and
one-hot gradient rows that must select rows of W exactly. Shapes span
several product tiles with ragged tails, and the real shapes of the 7B up
projection and of two 7B-stack projections at their full token count
(sampled token rows of dX and rows of S)."""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import BF16_TOL, device, rownorm_err, say, to_f64

pytestmark = pytest.mark.gpu


def _case(T, d, k, r, seed, dev, dy_std=1e-2):
    X, dY = inputs.random_case(seed, T, d, k, dtype=torch.bfloat16, dy_std=dy_std, outlier_cols=max(1, k // 100))
    g = inputs.generator("backward-W", seed, d, k)
    W = (torch.randn(d, k, generator=g) * 0.02).to(torch.bfloat16)
    return X.to(dev), dY.to(dev), W.to(dev)


def _run(m, X, dY, W, dev, mbs=1, placement=0):
    T = X.shape[0]
    ws = torch.empty(max(16, B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16)), dtype=torch.uint8, device=dev)
    S = torch.full((m.d, m.r), float("nan"), device=dev)
    dX = torch.full((T, m.k), float("nan"), dtype=torch.bfloat16, device=dev)
    dX0 = torch.full((T, m.k), float("nan"), dtype=torch.bfloat16, device=dev)
    for n in range(mbs):
        B.logra_sketch_project(m, X, ws)
        B.logra_backward_dx_sketch(m, dY, W, dX, S, n > 0, ws, opts=B.LaunchOpts(backward_fold=placement))
    B.logra_backward_dx(m, dY, W, dX0)
    torch.cuda.synchronize()
    return S, dX, dX0


SMALL = [
    # T, d, k, r, microbatches
    (300, 520, 264, 64, 1),
    (257, 136, 1000, 32, 2),
    (513, 1032, 520, 256, 1),
    (64, 8, 8, 32, 1),
    (1000, 8200, 136, 128, 2),
    (256, 256, 256, 256, 1),
    (520, 3000, 776, 256, 1),
    # d % 32 == 16 (a partial last chunk of the product's 32-wide ones) and
    # 11 chunks (three past a multiple of four), fewer tokens than one tile
    (200, 336, 392, 64, 1),
]


@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("T,d,k,r,mbs", SMALL)
def test_backward_dx_sketch_matches_oracle(T, d, k, r, mbs, placement):
    # placement 1: the fold in the product's launch; 2: the fold kernel after it
    dev = device()
    say("backward dx+sketch", T, d, k, r, mbs, "fold in the launch" if placement == 1 else "fold after")
    m = B.MatrixDesc(d, k, r, seed=4, step=T, matrix_id=k)
    X, dY, W = _case(T, d, k, r, 31 * T + d, dev)
    S, dX, dX0 = _run(m, X, dY, W, dev, mbs, placement)
    assert torch.equal(dX, dX0)
    ref = oracle.backward_dx_rows(to_f64(dY), to_f64(W))
    e_dx = rownorm_err(to_f64(dX), ref)
    A = oracle.sign_matrix(4, T, k, r, k)
    P = oracle.project(to_f64(X), A)
    S_ref = None
    for n in range(mbs):
        S_ref = oracle.sketch_rows(to_f64(dY), P, S_rows=S_ref, accumulate=n > 0)
    e_s = rownorm_err(to_f64(S), S_ref)
    say("  dX %.3e  S %.3e" % (e_dx, e_s))
    assert e_dx < BF16_TOL and e_s < BF16_TOL


def test_one_hot_gradient_rows_select_rows_of_W_exactly():
    dev = device()
    T, d, k, r = 300, 520, 264, 32
    m = B.MatrixDesc(d, k, r)
    picks = torch.from_numpy(np.random.default_rng(5).choice(d, T, replace=True))
    dY = torch.zeros(T, d, dtype=torch.bfloat16)
    dY[torch.arange(T), picks] = 1.0
    g = inputs.generator("backward-W", 0, d, k)
    W = (torch.randn(d, k, generator=g) * 0.02).to(torch.bfloat16)
    dX = torch.empty(T, k, dtype=torch.bfloat16, device=dev)
    B.logra_backward_dx(m, dY.to(dev), W.to(dev), dX)
    torch.cuda.synchronize()
    assert torch.equal(dX.cpu(), W[picks])


@pytest.mark.parametrize("d,k,ntok", [(18944, 3584, 48), (3584, 3584, 48), (3584, 18944, 24), (512, 3584, 48)])
def test_backward_dx_sketch_at_7b_shapes(d, k, ntok):
    # the 7B up projection (d = 18944, k = 3584) and the 7B stack's q, down
    # and k projections at 4096 tokens, with the library's choice of where the
    # fold runs (in the launch for the first three, after it for k): sampled
    # token rows of dX and rows of S
    dev = device()
    T, r = 4096, 256
    say("backward dx+sketch", T, d, k, r)
    wl = inputs.WORKLOADS["qwen7b_up"]
    spec = inputs.MatrixSpec("up", 0, d, k, 5)
    X = inputs.activations(wl, spec, 0, 0, device=dev)
    dY = inputs.output_grads(wl, spec, 0, 0, device=dev)
    W = inputs.weights(wl, spec, device=dev)
    m = B.MatrixDesc(d, k, r, seed=0, step=0, matrix_id=5)
    S, dX, dX0 = _run(m, X, dY, W, dev)
    assert torch.equal(dX, dX0)
    rng = np.random.default_rng(d + k)
    trows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, ntok, replace=False)]))
    srows = np.unique(np.concatenate([[0, d - 1], rng.choice(d, 256, replace=False)]))
    W_h = to_f64(W)
    ref_dx = oracle.backward_dx_rows(to_f64(dY[torch.from_numpy(trows).to(dev)]), W_h)
    e_dx = rownorm_err(to_f64(dX)[trows], ref_dx)
    A = oracle.sign_matrix(0, 0, 5, r, k)
    P = oracle.project_matmul(to_f64(X), A)
    S_ref = oracle.sketch_rows(to_f64(dY[:, torch.from_numpy(srows).to(dev)]), P)
    e_s = rownorm_err(to_f64(S)[srows], S_ref)
    say("  dX %.3e  S %.3e" % (e_dx, e_s))
    assert e_dx < BF16_TOL and e_s < BF16_TOL


def test_strided_operands_give_the_contiguous_result():
    # dY, W and dX as column slices of wider tensors (leading dimensions
    # past d and k, multiples of 8): the same bits as contiguous operands,
    # with the fold in the launch and after it
    dev = device()
    T, d, k, r = 300, 1032, 264, 64
    m = B.MatrixDesc(d, k, r, seed=6, step=1, matrix_id=2)
    X, dY, W = _case(T, d, k, r, 77, dev)
    dY_w = torch.zeros(T, d + 24, dtype=torch.bfloat16, device=dev)
    W_w = torch.zeros(d, k + 40, dtype=torch.bfloat16, device=dev)
    dY_w[:, :d] = dY
    W_w[:, :k] = W
    dYs, Ws = dY_w[:, :d], W_w[:, :k]
    for placement in (1, 2):
        say("backward dx strided", T, d, k, r, placement)
        S, dX, dX0 = _run(m, X, dY, W, dev, 1, placement)
        ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
        S_s = torch.full((d, r), float("nan"), device=dev)
        dX_w = torch.full((T, k + 16), float("nan"), dtype=torch.bfloat16, device=dev)
        B.logra_sketch_project(m, X, ws)
        B.logra_backward_dx_sketch(m, dYs, Ws, dX_w[:, :k], S_s, False, ws, opts=B.LaunchOpts(backward_fold=placement))
        torch.cuda.synchronize()
        assert torch.equal(dX_w[:, :k], dX)
        assert torch.isnan(dX_w[:, k:].float()).all()   # the columns past k are not written
        assert torch.equal(S_s, S)


def test_backward_errors_leave_outputs_untouched():
    dev = device()
    T, d, k, r = 64, 64, 128, 32
    m = B.MatrixDesc(d, k, r)
    X, dY, W = _case(T, d, k, r, 9, dev)
    dX = torch.zeros(T, k, dtype=torch.bfloat16, device=dev)
    with pytest.raises(B.LograError) as e:
        B.logra_backward_dx(m, dY.float(), W, dX)             # fp32 inputs: unsupported
    assert e.value.status == 2
    with pytest.raises(B.LograError) as e:
        B.logra_backward_dx(m, dY, W[:, 1:], dX)     # W not 16-byte aligned
    assert e.value.status == 1
    S = torch.zeros(d, r, device=dev)
    with pytest.raises(B.LograError) as e:
        B.logra_backward_dx_sketch(m, dY, W, dX, S, False, torch.empty(16, dtype=torch.uint8, device=dev))
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.count_nonzero(dX).item() == 0 and torch.count_nonzero(S).item() == 0
