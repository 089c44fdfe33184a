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
from gpu_util import (BF16_TOL, F32_TOL, bf16_w_check, device, f32, rel_err, rownorm_err, say,
                      to_f64, w_update_err)

pytestmark = pytest.mark.gpu


def _rows(d, n, seed):
    if n is None or n >= d:
        return np.arange(d)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, d - 1], rng.choice(d, n, replace=False)]))


def _code(dt):
    return B.LOGRA_BF16 if dt == torch.bfloat16 else B.LOGRA_F32


def _step_and_check(wl, spec, step, st, dev, mbs, T, tol, data_seed=0):
    """One optimizer step on the GPU and on the oracle (sampled rows st["rows"]);
    checks S, rowsq, v', the W update and the sqnorm identity. Each side
    carries its own state (W, v) from step to step; the oracle's W is kept at
    the stored dtype (rounded to bf16 for bf16 W), as the step stores it."""
    d, k, r = spec.d, spec.k, wl.r
    rows = st["rows"]
    m = B.MatrixDesc(d, k, r, seed=data_seed, step=step, matrix_id=spec.matrix_id)
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
    e_s = rownorm_err(to_f64(S)[rows], S_ref)

    beta2, eps, lr = wl.beta2, wl.eps, wl.lr
    scale = inputs.step_scale(wl, spec, step, data_seed)
    hp = dict(beta2=f32(beta2), eps=f32(eps), lr=f32(lr), scale=f32(scale))
    compute = _code(wl.act_dtype)
    W, v, W32 = st["W"], st["v"], st["W32"]
    rowsq = torch.empty(d, dtype=torch.float32, device=dev)
    v_new = torch.empty(d, dtype=torch.float32, device=dev)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    B.logra_update_sqnorm(m, compute, S, v, beta2, eps, v_new, sq, rowsq)
    torch.cuda.synchronize()
    # sqnorm identity over all rows, from the GPU's own rowsq and v (a property
    # of the GPU outputs; no oracle input)
    rowsq_h, v_old_h = to_f64(rowsq), to_f64(v)
    vn = hp["beta2"] * v_old_h + (1 - hp["beta2"]) * rowsq_h / k
    ident = float((rowsq_h / (np.sqrt(vn) + hp["eps"]) ** 2).sum())
    e_ident = abs(sq.item() / ident - 1)

    ref = oracle.rowadam_rows(S_ref, A, st["v_ref"], st["W_ref"], **hp)
    e_rq = rel_err(rowsq_h[rows], ref["rowsq"])
    B.logra_rowadam_apply(m, compute, S, v_new, W, lr, scale, eps)
    if W32 is not None:
        B.logra_rowadam_apply(m, compute, S, v_new, W32, lr, scale, eps)
    torch.cuda.synchronize()
    e_v = rel_err(to_f64(v_new)[rows], ref["v_new"])
    st["v"] = v_new   # the update was applied: v' is the next step's v
    W_new = to_f64(W)[rows]
    if W.dtype == torch.bfloat16:
        w_ok, _, st["allow"] = bf16_w_check(W_new, ref["W_new"], st["W_ref"], prior=st.get("allow"))
        ref32 = oracle.rowadam_rows(S_ref, A, st["v_ref"], st["W32_ref"], **hp)
        e_w = w_update_err(to_f64(W32)[rows], ref32["W_new"], st["W32_ref"])
        st["W32_ref"] = ref32["W_new"]
        st["W_ref"] = torch.from_numpy(ref["W_new"]).to(torch.bfloat16).double().numpy()
    else:
        w_ok = True
        e_w = w_update_err(W_new, ref["W_new"], st["W_ref"])
        st["W_ref"] = ref["W_new"]
    st["v_ref"] = ref["v_new"]
    say("  %s step %d: S %.2e rowsq %.2e v %.2e dW %.2e sqnorm-identity %.2e W-bf16 %s"
        % (spec.name, step, e_s, e_rq, e_v, e_w, e_ident, w_ok))
    assert e_s < tol and e_rq < tol and e_v < tol and e_w < tol and e_ident < tol and w_ok
    return st


def _init_state(wl, spec, dev, shadow, nrows):
    """GPU state from the input generator, and the oracle's copy of the same
    generated values on the sampled rows."""
    W_h = inputs.weights(wl, spec)
    v_h = inputs.second_moment(wl, spec)
    rows = _rows(spec.d, nrows, spec.matrix_id)
    st = {"rows": rows, "W": W_h.to(dev), "v": v_h.to(dev), "W32": None,
          "W_ref": W_h.double().numpy()[rows], "v_ref": v_h.double().numpy()[rows],
          "W32_ref": None}
    if shadow and W_h.dtype == torch.bfloat16:
        st["W32"] = W_h.float().to(dev)
        st["W32_ref"] = W_h.double().numpy()[rows]
    return st


def test_tiny_fp32_workload_full():
    dev = device()
    wl = inputs.WORKLOADS["tiny_fp32"]
    spec = wl.matrices[0]
    say("workload tiny_fp32", spec)
    st = _init_state(wl, spec, dev, shadow=False, nrows=None)
    _step_and_check(wl, spec, 0, st, dev, wl.microbatches, wl.tokens, F32_TOL)


def test_qwen15b_set_all_projections():
    dev = device()
    wl = inputs.WORKLOADS["qwen1.5b_set"]
    for spec in wl.matrices:
        say("workload qwen1.5b_set", spec)
        st = _init_state(wl, spec, dev, shadow=True, nrows=256)
        _step_and_check(wl, spec, 0, st, dev, 2, wl.tokens, BF16_TOL)


def test_qwen7b_up_two_steps_full_microbatches():
    # The benchmarked workload: 16 microbatches of 4096 tokens per step, A
    # redrawn at the next step, W and v carried over.
    dev = device()
    wl = inputs.WORKLOADS["qwen7b_up"]
    spec = wl.matrices[0]
    st = _init_state(wl, spec, dev, shadow=True, nrows=512)
    for step in range(2):
        say("workload qwen7b_up step", step)
        st = _step_and_check(wl, spec, step, st, dev, wl.microbatches, wl.tokens, BF16_TOL)


@pytest.mark.parametrize("name", ["qwen7b_28layer", "27b_64layer"])
def test_one_layer_of_large_stacks(name):
    # Every projection shape of the 28-layer 7B and 64-layer 27B stacks (one
    # layer, one microbatch of the full token count).
    dev = device()
    wl = inputs.WORKLOADS[name]
    for spec in wl.matrices[:7]:
        say("workload", name, spec)
        st = _init_state(wl, spec, dev, shadow=True, nrows=256)
        _step_and_check(wl, spec, 0, st, dev, 1, wl.tokens, BF16_TOL)
