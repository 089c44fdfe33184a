"""Workload-level GPU parity: whole optimizer steps (all microbatches, pass 1,
pass 2) at the real shapes of the five workloads, against the oracle.

Rows of S, Ghat and W are independent once P = X A^T is known, so the
oracle computes P in full and only a seeded sample of rows (plus the first
and last) of everything else; that comparison is exact in what it covers.
The full-matrix sqnorm is checked through the identity sqnorm = sum_i rowsq_i
u_i^2 (u from the GPU's rowsq and v) and the sampled rowsq against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import BF16_TOL, F32_TOL, bf16_ulp, device, rel_err, rownorm_err, say, to_f64

pytestmark = pytest.mark.gpu


def _rows(d, n, seed):
    if n is None or n >= d:
        return np.arange(d)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, d - 1], rng.choice(d, n, replace=False)]))


def _code(dt):
    return B.LOGRA_BF16 if dt == torch.bfloat16 else B.LOGRA_F32


def _step_and_check(wl, spec, step, state, dev, mbs, T, nrows, tol, data_seed=0):
    """One optimizer step on the GPU and on the oracle (sampled rows); checks
    S, rowsq, v', the W update and the sqnorm identity; returns the new state."""
    d, k, r = spec.d, spec.k, wl.r
    m = B.MatrixDesc(d, k, r, seed=data_seed, step=step, matrix_id=spec.matrix_id)
    rows = _rows(d, nrows, 1000 * step + spec.matrix_id)
    A = oracle.sign_matrix(data_seed, step, spec.matrix_id, r, k)
    S = torch.empty(d, r, dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, B.logra_sketch_workspace_bytes(m, T, _code(wl.act_dtype))),
                     dtype=torch.uint8, device=dev)
    S_ref = None
    for mb in range(mbs):
        X = inputs.activations(wl, spec, step, mb, T=T, data_seed=data_seed)
        dY = inputs.output_grads(wl, spec, step, mb, T=T, data_seed=data_seed)
        B.logra_sketch_accumulate(m, X.to(dev), dY.to(dev), S, accumulate=mb > 0, ws=ws)
        P = oracle.project(X.double().numpy(), A)
        S_ref = oracle.sketch_rows(dY.double().numpy(), P, rows=rows, S_rows=S_ref,
                                   accumulate=mb > 0)
    torch.cuda.synchronize()
    S_h = to_f64(S)
    e_s = rownorm_err(S_h[rows], S_ref)

    W, v, W32 = state
    beta2, eps, lr = wl.beta2, wl.eps, wl.lr
    scale = inputs.step_scale(wl, spec, step, data_seed)
    compute = _code(wl.act_dtype)
    rowsq = torch.empty(d, dtype=torch.float32, device=dev)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    B.logra_update_sqnorm(m, compute, S, v, beta2, eps, rowsq, sq)
    torch.cuda.synchronize()
    rowsq_h = to_f64(rowsq)
    v_old = to_f64(v)
    # sqnorm identity over all rows, from the GPU's own rowsq and v
    vn = beta2 * v_old + (1 - beta2) * rowsq_h / k
    ident = float((rowsq_h / (np.sqrt(vn) + eps) ** 2).sum())
    e_ident = abs(sq.item() / ident - 1)
    W_old = to_f64(W)[rows]
    W32_old = to_f64(W32)[rows] if W32 is not None else None
    ref = oracle.rowadam_rows(S_ref, A, v_old[rows], W_old, beta2=beta2, eps=eps, lr=lr, scale=scale)
    e_rq = rel_err(rowsq_h[rows], ref["rowsq"])
    B.logra_rowadam_apply(m, compute, S, v, rowsq, W, lr, scale, beta2, eps)
    if W32 is not None:
        v_sh = torch.from_numpy(v_old).float().to(dev)
        B.logra_rowadam_apply(m, compute, S, v_sh, rowsq, W32, lr, scale, beta2, eps)
    torch.cuda.synchronize()
    e_v = rel_err(to_f64(v)[rows], ref["v_new"])
    W_new = to_f64(W)[rows]
    if W.dtype == torch.bfloat16:
        W_ref_b = torch.from_numpy(ref["W_new"]).to(torch.bfloat16).double().numpy()
        w_ok = bool(np.all(np.abs(W_new - W_ref_b) <= bf16_ulp(W_ref_b)))
        ref32 = oracle.rowadam_rows(S_ref, A, v_old[rows], W32_old, beta2=beta2, eps=eps, lr=lr,
                                    scale=scale)
        e_w = rownorm_err(to_f64(W32)[rows] - W32_old, ref32["W_new"] - W32_old)
    else:
        w_ok = True
        e_w = rownorm_err(W_new - W_old, ref["W_new"] - W_old)
    say("  %s step %d: S %.2e rowsq %.2e v %.2e dW %.2e sqnorm-identity %.2e W-ulp %s"
        % (spec.name, step, e_s, e_rq, e_v, e_w, e_ident, w_ok))
    assert e_s < tol and e_rq < tol and e_v < tol and e_w < tol and e_ident < tol and w_ok
    return W, v, W32


def _init_state(wl, spec, dev, shadow):
    W = inputs.weights(wl, spec).to(dev)
    v = inputs.second_moment(wl, spec).to(dev)
    W32 = W.float().clone() if (shadow and W.dtype == torch.bfloat16) else None
    return W, v, W32


def test_tiny_fp32_workload_full():
    dev = device()
    wl = inputs.WORKLOADS["tiny_fp32"]
    spec = wl.matrices[0]
    say("workload tiny_fp32", spec)
    state = _init_state(wl, spec, dev, shadow=False)
    _step_and_check(wl, spec, 0, state, dev, wl.microbatches, wl.tokens, None, F32_TOL)


def test_qwen15b_set_all_projections():
    dev = device()
    wl = inputs.WORKLOADS["qwen1.5b_set"]
    for spec in wl.matrices:
        say("workload qwen1.5b_set", spec)
        state = _init_state(wl, spec, dev, shadow=True)
        _step_and_check(wl, spec, 0, state, dev, 2, wl.tokens, 256, BF16_TOL)


def test_qwen7b_up_two_steps_full_microbatches():
    # The benchmarked workload: 16 microbatches of 4096 tokens per step, A
    # redrawn at the next step, W and v carried over.
    dev = device()
    wl = inputs.WORKLOADS["qwen7b_up"]
    spec = wl.matrices[0]
    state = _init_state(wl, spec, dev, shadow=True)
    for step in range(2):
        say("workload qwen7b_up step", step)
        state = _step_and_check(wl, spec, step, state, dev, wl.microbatches, wl.tokens, 512, BF16_TOL)


@pytest.mark.parametrize("name", ["qwen7b_28layer", "27b_64layer"])
def test_one_layer_of_large_stacks(name):
    # Every projection shape of the 28-layer 7B and 64-layer 27B stacks (one
    # layer, one microbatch of the full token count).
    dev = device()
    wl = inputs.WORKLOADS[name]
    for spec in wl.matrices[:7]:
        say("workload", name, spec)
        state = _init_state(wl, spec, dev, shadow=True)
        _step_and_check(wl, spec, 0, state, dev, 1, wl.tokens, 256, BF16_TOL)
