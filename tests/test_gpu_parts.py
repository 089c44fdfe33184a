"""GPU parity of the fold that holds a step's sketch in parts
(logra_sketch_fold_parts) through the C ABI against the oracle: S after the
step's last microbatch per row (normwise) at 2e-2, the sum S + parts after a
middle microbatch at the same bound, bitwise repeatability, the work splits
that use parts (two members per tile, more members per tile) and the one that
needs none (short token counts), a one-microbatch step, microbatches folded
by logra_sketch_fold and logra_backward_dx_sketch between parts calls, and the
7B up projection at its full token count (sampled rows)."""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import BF16_TOL, device, rownorm_err, say, to_f64

pytestmark = pytest.mark.gpu

FIRST, LAST = B.LOGRA_FOLD_FIRST, B.LOGRA_FOLD_LAST


def _inputs(T, d, k, n, seed, dev):
    Xs, dYs = [], []
    for i in range(n):
        X, dY = inputs.random_case(seed + 101 * i, T, d, k, dtype=torch.bfloat16, dy_std=1e-2,
                                   outlier_cols=max(1, k // 100))
        Xs.append(X.to(dev))
        dYs.append(dY.to(dev))
    return Xs, dYs


def _ref(m, Xs, dYs, upto=None, rows=None):
    A = oracle.sign_matrix(m.seed, m.step, m.matrix_id, m.r, m.k)
    S = None
    for n, (X, dY) in enumerate(zip(Xs, dYs)):
        if upto is not None and n >= upto:
            break
        dy = to_f64(dY) if rows is None else to_f64(dY[:, torch.from_numpy(rows).to(dY.device)])
        S = oracle.sketch_rows(dy, oracle.project(to_f64(X), A), S_rows=S, accumulate=n > 0)
    return S


def _parts_run(m, Xs, dYs, dev, check_after=None):
    """FIRST, middles, LAST over the microbatches; returns S and, when asked,
    S + parts (fp64, host) after microbatch check_after."""
    T = Xs[0].shape[0]
    n = len(Xs)
    ws = torch.empty(max(16, B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16)), dtype=torch.uint8, device=dev)
    pb = B.logra_sketch_parts_bytes(m, T, B.LOGRA_BF16)
    parts = torch.full((max(1, pb // 4),), float("nan"), device=dev) if pb else None
    S = torch.full((m.d, m.r), float("nan"), device=dev)
    mid_sum = None
    for i in range(n):
        phase = (FIRST if i == 0 else 0) | (LAST if i == n - 1 else 0)
        B.logra_sketch_project(m, Xs[i], ws)
        B.logra_sketch_fold_parts(m, dYs[i], S, parts, phase, ws)
        if check_after is not None and i == check_after:
            torch.cuda.synchronize()
            mid_sum = to_f64(S)
            if parts is not None:
                for q in range(pb // (4 * m.d * m.r)):
                    mid_sum = mid_sum + to_f64(parts[q * m.d * m.r:(q + 1) * m.d * m.r].view(m.d, m.r))
    torch.cuda.synchronize()
    return S, mid_sum, pb


CASES = [
    # T, d, k, r, microbatches; the plan each exercises
    (300, 8200, 136, 64, 3),     # two members per tile (d >= 8192): one part
    (1000, 520, 264, 128, 3),    # small d: three members per tile, two parts
    (2052, 3592, 136, 256, 2),   # small d, four members per tile, ragged T
    (100, 8200, 136, 32, 3),     # four token steps: one member per tile, no parts
    (513, 16392, 72, 256, 2),    # tall tiles, two members, ragged d
]


@pytest.mark.parametrize("T,d,k,r,n", CASES)
def test_fold_parts_matches_oracle(T, d, k, r, n):
    dev = device()
    say("fold_parts", T, d, k, r, n)
    m = B.MatrixDesc(d, k, r, seed=3, step=T, matrix_id=d)
    Xs, dYs = _inputs(T, d, k, n, 7 * T + d, dev)
    S, mid, pb = _parts_run(m, Xs, dYs, dev, check_after=n - 2)
    e_mid = rownorm_err(mid, _ref(m, Xs, dYs, upto=n - 1))
    e = rownorm_err(to_f64(S), _ref(m, Xs, dYs))
    say("  parts bytes %d  S+parts after %d: %.3e  S at the end: %.3e" % (pb, n - 1, e_mid, e))
    assert e_mid < BF16_TOL and e < BF16_TOL


def test_fold_parts_is_bitwise_repeatable():
    dev = device()
    T, d, k, r, n = 300, 8200, 136, 256, 3
    m = B.MatrixDesc(d, k, r, seed=1, step=2, matrix_id=3)
    Xs, dYs = _inputs(T, d, k, n, 11, dev)
    S1, _, _ = _parts_run(m, Xs, dYs, dev)
    S2, _, _ = _parts_run(m, Xs, dYs, dev)
    assert torch.equal(S1, S2)


def test_one_microbatch_step():
    dev = device()
    T, d, k, r = 520, 8200, 264, 128
    m = B.MatrixDesc(d, k, r, seed=5, step=0, matrix_id=1)
    Xs, dYs = _inputs(T, d, k, 1, 13, dev)
    S, _, pb = _parts_run(m, Xs, dYs, dev)
    assert pb > 0
    assert rownorm_err(to_f64(S), _ref(m, Xs, dYs)) < BF16_TOL


def test_other_folds_between_parts_calls():
    # microbatch 1 through logra_sketch_fold, microbatch 2 through
    # logra_backward_dx_sketch, both with accumulate = 1: they add to S alone
    dev = device()
    T, d, k, r, n = 300, 8200, 264, 64, 4
    m = B.MatrixDesc(d, k, r, seed=2, step=9, matrix_id=4)
    Xs, dYs = _inputs(T, d, k, n, 17, dev)
    g = inputs.generator("parts-W", 0, d, k)
    W = (torch.randn(d, k, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    dX = torch.empty(T, k, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    parts = torch.empty(B.logra_sketch_parts_bytes(m, T, B.LOGRA_BF16) // 4, device=dev)
    S = torch.full((d, r), float("nan"), device=dev)
    for i in range(n):
        B.logra_sketch_project(m, Xs[i], ws)
        if i == 1:
            B.logra_sketch_fold(m, dYs[i], S, True, ws)
        elif i == 2:
            B.logra_backward_dx_sketch(m, dYs[i], W, dX, S, True, ws)
        else:
            B.logra_sketch_fold_parts(m, dYs[i], S, parts, FIRST if i == 0 else LAST, ws)
    torch.cuda.synchronize()
    assert rownorm_err(to_f64(S), _ref(m, Xs, dYs)) < BF16_TOL


def test_fold_parts_at_the_7b_up_shape():
    # d = 18944, k = 3584, r = 256, 4096 tokens, three microbatches (first,
    # middle, last): sampled rows of S, plus the first and last row
    dev = device()
    T, d, k, r = 4096, 18944, 3584, 256
    say("fold_parts 7B up", T, d, k, r)
    wl = inputs.WORKLOADS["qwen7b_up"]
    spec = inputs.MatrixSpec("up", 0, d, k, 5)
    Xs = [inputs.activations(wl, spec, 0, mb, device=dev) for mb in range(3)]
    dYs = [inputs.output_grads(wl, spec, 0, mb, device=dev) for mb in range(3)]
    m = B.MatrixDesc(d, k, r, seed=0, step=0, matrix_id=5)
    S, _, pb = _parts_run(m, Xs, dYs, dev)
    assert pb == d * r * 4
    rows = np.unique(np.concatenate([[0, d - 1], np.random.default_rng(1).choice(d, 256, replace=False)]))
    A = oracle.sign_matrix(0, 0, 5, r, k)
    S_ref = None
    for i in range(3):
        P = oracle.project_matmul(to_f64(Xs[i]), A)
        S_ref = oracle.sketch_rows(to_f64(dYs[i][:, torch.from_numpy(rows).to(dev)]), P, S_rows=S_ref,
                                   accumulate=i > 0)
    e = rownorm_err(to_f64(S)[rows], S_ref)
    say("  S %.3e" % e)
    assert e < BF16_TOL
