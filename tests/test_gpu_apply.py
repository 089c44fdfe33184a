"""GPU parity of the apply passes: logra_update_sqnorm (pass 1) and
logra_rowadam_apply (pass 2) through the C ABI against the CPU oracle.

S, v and W are seeded inputs shared by both sides. rowsq, v', sqnorm and the
W update are compared at 2e-2 (bf16 MFMA compute) or 1e-5 (fp32 compute);
bf16 W within one bf16 ulp plus the update tolerance (see gpu_util), and an
fp32-W shadow run of the same step.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import (BF16_TOL, F32_TOL, bf16_w_check, device, f32, rel_err, say, to_f64,
                      w_update_err)

pytestmark = pytest.mark.gpu


def _state(seed, d, k, r, s_std=1e-2):
    g = inputs.generator("apply-state", seed, d, k, r)
    S = torch.randn(d, r, generator=g) * s_std
    v = 1e-10 + torch.rand(d, generator=g) * 1e-6
    W = torch.randn(d, k, generator=g) * 0.02
    return S, v, W


def _run(m, compute, S, v, W, lr, scale, beta2, eps, dev, opts=None):
    S_d, v_d, W_d = S.to(dev), v.clone().to(dev), W.clone().to(dev)
    v_new = torch.empty(m.d, dtype=torch.float32, device=dev)
    rowsq = torch.empty(m.d, dtype=torch.float32, device=dev)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    B.logra_update_sqnorm(m, compute, S_d, v_d, beta2, eps, v_new, sq, rowsq)
    torch.cuda.synchronize()
    rowsq_h, sq_h = rowsq.cpu(), sq.item()
    B.logra_rowadam_apply(m, compute, S_d, v_new, W_d, lr, scale, eps, opts=opts)
    torch.cuda.synchronize()
    # pass 1 leaves v as it was
    assert torch.equal(v_d.cpu(), v)
    return rowsq_h, sq_h, v_new.cpu(), W_d.cpu()


APPLY_CASES = [
    # d, k, r
    # (1000, 4104, 256): more 256-row x 64-column units than workgroups, so a
    # workgroup walks several units, crosses row tiles, and ends on the
    # partial last row tile and column tile
    (1000, 4104, 256),
    (64, 128, 32),
    (200, 520, 64),
    (136, 1000, 128),
    (520, 1544, 256),
    (8, 8, 256),
    (1032, 4104, 256),
    # pass 1 with 3 row blocks per workgroup and a ragged last workgroup
    (8200, 136, 256),
    # pass 1 with 258 workgroups of 8 row blocks: the last one to arrive adds
    # more partials than it has threads
    (33000, 72, 64),
]


@pytest.mark.parametrize("d,k,r", APPLY_CASES)
@pytest.mark.parametrize("wdt", [torch.float32, torch.bfloat16])
def test_apply_bf16_compute_matches_oracle(d, k, r, wdt):
    dev = device()
    say("apply bf16", d, k, r, wdt)
    m = B.MatrixDesc(d, k, r, seed=2, step=d, matrix_id=k)
    S, v, W = _state(d + k, d, k, r)
    W = W.to(wdt)
    lr, scale, beta2, eps = 1e-3, 0.8, 0.999, 1e-8
    rowsq, sq, v_new, W_new = _run(m, B.LOGRA_BF16, S, v, W, lr, scale, beta2, eps, dev)
    A = oracle.sign_matrix(2, d, k, r, k)
    ref = oracle.rowadam_rows(S.double().numpy(), A, v.double().numpy(), W.double().numpy(),
                              beta2=f32(beta2), eps=f32(eps), lr=f32(lr), scale=f32(scale))
    e_rq = rel_err(rowsq.double().numpy(), ref["rowsq"])
    e_v = rel_err(v_new.double().numpy(), ref["v_new"])
    e_sq = abs(sq / ref["sqnorm"] - 1)
    say("  rowsq %.2e v %.2e sqnorm %.2e" % (e_rq, e_v, e_sq))
    assert e_rq < BF16_TOL and e_v < BF16_TOL and e_sq < BF16_TOL
    W0 = W.double().numpy()
    if wdt == torch.float32:
        e_w = w_update_err(W_new.double().numpy(), ref["W_new"], W0)
        say("  dW %.2e" % e_w)
        assert e_w < BF16_TOL
    else:
        ok, worst, _ = bf16_w_check(W_new.double().numpy(), ref["W_new"], W0)
        say("  bf16 W worst error / allowed %.3f" % worst)
        assert ok


@pytest.mark.parametrize("d,k,r", [(1000, 4104, 256), (200, 520, 64), (8200, 136, 32)])
def test_prepared_pass1_equals_one_call(d, k, r):
    # The Gram matrix built ahead on a second stream (ordered by an event),
    # then the rest of pass 1: bit-identical to logra_update_sqnorm.
    dev = device()
    say("pass 1 prepared", d, k, r)
    m = B.MatrixDesc(d, k, r, seed=8, step=d, matrix_id=r)
    S, v, _ = _state(11 * d + r, d, k, r)
    S, v = S.to(dev), v.to(dev)
    outs = []
    for prepared in (False, True):
        v_new = torch.empty(d, device=dev)
        rowsq = torch.empty(d, device=dev)
        sq = torch.empty(1, device=dev)
        ws = torch.empty(B.logra_sqnorm_workspace_bytes(m, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
        if prepared:
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(torch.cuda.current_stream())
            B.logra_sqnorm_prepare(m, B.LOGRA_BF16, ws, side)
            torch.cuda.current_stream().wait_stream(side)
            B.logra_update_sqnorm_prepared(m, B.LOGRA_BF16, S, v, 0.999, 1e-8, v_new, sq, ws, rowsq)
        else:
            B.logra_update_sqnorm(m, B.LOGRA_BF16, S, v, 0.999, 1e-8, v_new, sq, rowsq, ws)
        torch.cuda.synchronize()
        outs.append((v_new.cpu(), rowsq.cpu(), sq.cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,k,r", [(1000, 4104, 256), (4608, 3592, 256), (8200, 136, 256)])
def test_apply_concurrency_hint_keeps_parity(d, k, r):
    # With an apply concurrency of 3 pass 2 of a matrix of at least 1024
    # 256 x 64 tiles (4608 x 3592: 18 x 57) runs on 128 workgroups, and in
    # 256-row tiles from half as many units; smaller ones keep the default
    # grid. W matches the oracle to the same bound either way.
    dev = device()
    say("apply concurrency 3", d, k, r)
    m = B.MatrixDesc(d, k, r, seed=6, step=d, matrix_id=k)
    S, v, W = _state(7 * d + k, d, k, r)
    W = W.to(torch.bfloat16)
    lr, scale, beta2, eps = 1e-3, 0.8, 0.999, 1e-8
    _, _, v_new, W_new = _run(m, B.LOGRA_BF16, S, v, W, lr, scale, beta2, eps, dev,
                              opts=B.LaunchOpts(apply_concurrency=3))
    A = oracle.sign_matrix(6, d, k, r, k)
    ref = oracle.rowadam_rows(S.double().numpy(), A, v.double().numpy(), W.double().numpy(),
                              beta2=f32(beta2), eps=f32(eps), lr=f32(lr), scale=f32(scale))
    assert rel_err(v_new.double().numpy(), ref["v_new"]) < BF16_TOL
    ok, worst, _ = bf16_w_check(W_new.double().numpy(), ref["W_new"], W.double().numpy())
    say("  bf16 W worst error / allowed %.3f" % worst)
    assert ok


@pytest.mark.parametrize("d,k,r", [(256, 512, 32), (45, 130, 20), (300, 65, 1), (64, 256, 100),
                                   (17, 9, 1024)])
def test_apply_f32_compute_matches_oracle(d, k, r):
    dev = device()
    say("apply f32", d, k, r)
    m = B.MatrixDesc(d, k, r, seed=4, step=1, matrix_id=r)
    S, v, W = _state(3 * d + r, d, k, r)
    lr, scale, beta2, eps = 1e-3, 1.0, 0.999, 1e-8
    rowsq, sq, v_new, W_new = _run(m, B.LOGRA_F32, S, v, W, lr, scale, beta2, eps, dev)
    A = oracle.sign_matrix(4, 1, r, r, k)
    ref = oracle.rowadam_rows(S.double().numpy(), A, v.double().numpy(), W.double().numpy(),
                              beta2=f32(beta2), eps=f32(eps), lr=f32(lr), scale=f32(scale))
    e_rq = rel_err(rowsq.double().numpy(), ref["rowsq"])
    e_v = rel_err(v_new.double().numpy(), ref["v_new"])
    e_sq = abs(sq / ref["sqnorm"] - 1)
    W0 = W.double().numpy()
    e_w = w_update_err(W_new.double().numpy(), ref["W_new"], W0)
    say("  rowsq %.2e v %.2e sqnorm %.2e dW %.2e" % (e_rq, e_v, e_sq, e_w))
    assert max(e_rq, e_v, e_sq, e_w) < F32_TOL


@pytest.mark.parametrize("compute", [B.LOGRA_BF16, B.LOGRA_F32])
def test_one_hot_S_exposes_signs_through_apply(compute):
    # S row i = e_{i mod r}: Ghat row i = c * Sigma[i mod r], rowsq = k/r exactly,
    # and the sign of each W update is the sign of that Sigma entry.
    dev = device()
    d, k, r = 320, 392, 64
    m = B.MatrixDesc(d, k, r, seed=8, step=8, matrix_id=8)
    S = torch.zeros(d, r)
    S[torch.arange(d), torch.arange(d) % r] = 1.0
    v = torch.zeros(d)
    W = torch.zeros(d, k)
    rowsq, sq, v_new, W_new = _run(m, compute, S, v, W, 1.0, 1.0, 0.0, 0.0, dev)
    assert torch.all(rowsq == k / r)
    A = oracle.sign_matrix(8, 8, 8, r, k)
    expect = -np.sign(A[np.arange(d) % r])
    assert np.array_equal(np.sign(W_new.double().numpy()), expect)


def test_scale_zero_and_beta2_one_special_cases():
    dev = device()
    d, k, r = 128, 256, 256
    m = B.MatrixDesc(d, k, r, 1, 1, 1)
    S, v, W = _state(9, d, k, r)
    for wdt in (torch.float32, torch.bfloat16):
        Wt = W.to(wdt)
        _, _, v_new, W_new = _run(m, B.LOGRA_BF16, S, v, Wt, 1e-3, 0.0, 0.999, 1e-8, dev)
        assert torch.equal(W_new, Wt)
    _, _, v_new, _ = _run(m, B.LOGRA_BF16, S, v, W, 1e-3, 1.0, 1.0, 1e-8, dev)
    assert torch.equal(v_new, v)


def test_apply_deterministic_and_nan_propagates():
    dev = device()
    d, k, r = 256, 1024, 256
    m = B.MatrixDesc(d, k, r, 5, 5, 5)
    S, v, W = _state(11, d, k, r)
    a = _run(m, B.LOGRA_BF16, S, v, W, 1e-3, 1.0, 0.99, 1e-8, dev)
    b = _run(m, B.LOGRA_BF16, S, v, W, 1e-3, 1.0, 0.99, 1e-8, dev)
    assert torch.equal(a[0], b[0]) and a[1] == b[1] and torch.equal(a[3], b[3])
    S[7, 3] = float("nan")
    rowsq, sq, _, _ = _run(m, B.LOGRA_BF16, S, v, W, 1e-3, 1.0, 0.99, 1e-8, dev)
    assert np.isnan(sq) and torch.isnan(rowsq[7]) and not torch.isnan(rowsq[8])


@pytest.mark.parametrize("wdt", [torch.bfloat16, torch.float32])
def test_policy_sync_replica_matches_trainer(wdt):
    # A rollout worker's copy of W is brought up to date from the sketch alone:
    # it receives (S, v', the matrix's seed/step/id, lr * scale, eps) instead of
    # W or a dense update, and pass 2 rebuilds the same update there. The
    # replica must equal the trainer's W bit for bit, and both must match the
    # oracle's RowAdam step (beta2 = 1 on v' reproduces the update from v').
    dev = device()
    d, k, r = 1032, 4104, 256
    m = B.MatrixDesc(d, k, r, seed=13, step=4, matrix_id=6)
    S, v, W = _state(17, d, k, r)
    W = W.to(wdt)
    lr, scale, beta2, eps = 1e-3, 0.6, 0.999, 1e-8
    S_d, v_d = S.to(dev), v.to(dev)
    v_new = torch.empty(d, dtype=torch.float32, device=dev)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    B.logra_update_sqnorm(m, B.LOGRA_BF16, S_d, v_d, beta2, eps, v_new, sq)
    W_trainer, W_replica = W.clone().to(dev), W.clone().to(dev)
    B.logra_rowadam_apply(m, B.LOGRA_BF16, S_d, v_new, W_trainer, lr, scale, eps)
    # the message: S and v' (copied, as a transfer would), plus scalars
    msg_S, msg_v = S_d.clone(), v_new.clone()
    B.logra_rowadam_apply(B.MatrixDesc(d, k, r, seed=13, step=4, matrix_id=6), B.LOGRA_BF16,
                          msg_S, msg_v, W_replica, lr, scale, eps)
    torch.cuda.synchronize()
    assert torch.equal(W_trainer.cpu(), W_replica.cpu())
    msg_bytes = (msg_S.numel() + msg_v.numel()) * 4
    say("  policy sync: %d bytes instead of %d (W)" % (msg_bytes, W.numel() * W.element_size()))
    assert msg_bytes * 3 < W.numel() * W.element_size()
    A = oracle.sign_matrix(13, 4, 6, r, k)
    ref = oracle.rowadam_rows(S.double().numpy(), A, to_f64(v_new), W.double().numpy(),
                              beta2=1.0, eps=f32(eps), lr=f32(lr), scale=f32(scale))
    W0 = W.double().numpy()
    if wdt == torch.float32:
        assert w_update_err(to_f64(W_replica), ref["W_new"], W0) < BF16_TOL
    else:
        ok, _, _ = bf16_w_check(to_f64(W_replica), ref["W_new"], W0)
        assert ok


@pytest.mark.parametrize("compute", [B.LOGRA_BF16, B.LOGRA_F32])
def test_rowsq_output_is_optional(compute):
    # rowsq == NULL: the same v' and sqnorm, bit for bit, as with rowsq requested
    dev = device()
    d, k, r = 1032, 1544, 256 if compute == B.LOGRA_BF16 else 48
    m = B.MatrixDesc(d, k, r, 6, 2, 9)
    S, v, _ = _state(23, d, k, r)
    S_d, v_d = S.to(dev), v.to(dev)
    outs = []
    for want_rowsq in (True, False):
        v_new = torch.empty(d, device=dev)
        sq = torch.empty(1, device=dev)
        rowsq = torch.empty(d, device=dev) if want_rowsq else None
        B.logra_update_sqnorm(m, compute, S_d, v_d, 0.999, 1e-8, v_new, sq, rowsq)
        torch.cuda.synchronize()
        outs.append((v_new.cpu(), sq.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_controller_scale_through_the_gpu_update_meets_the_budget():
    # f1 end to end on the hot path: sqnorms from pass 1 on the GPU, the
    # library's host controller picks gamma for a budget a quarter of the
    # predicted KL, pass 2 applies lr * gamma; the realised 1/2 phi ||dW||^2
    # of the GPU's fp32 W update (over three matrices) must equal the budget
    # within the bf16-compute tolerance, and gamma = 1/2 exactly.
    dev = device()
    lr, phi, beta2, eps = 2e-3, 0.5, 0.999, 1e-8
    shapes = [(520, 1544, 256), (1032, 4104, 256), (200, 520, 64)]
    mats, sqs = [], []
    for idx, (d, k, r) in enumerate(shapes):
        m = B.MatrixDesc(d, k, r, 7, 11, idx)
        S, v, W = _state(31 + idx, d, k, r)
        S_d, v_d = S.to(dev), v.to(dev)
        v_new = torch.empty(d, device=dev)
        sq = torch.empty(1, device=dev)
        B.logra_update_sqnorm(m, B.LOGRA_BF16, S_d, v_d, beta2, eps, v_new, sq)
        mats.append((m, S_d, v_new, W.to(dev)))
        sqs.append(sq)
    torch.cuda.synchronize()
    sq_h = [float(q.item()) for q in sqs]
    _, kl0, _ = B.logra_kl_step_scale(sq_h, lr, phi, 1e30)
    delta = 0.25 * kl0
    scales, kl_pred, kl_after = B.logra_kl_step_scale(sq_h, lr, phi, delta)
    assert np.allclose(scales, 0.5, rtol=1e-6) and abs(kl_after / delta - 1) < 1e-9
    dw2 = 0.0
    for (m, S_d, v_new, W_d), sc in zip(mats, scales):
        W0 = W_d.clone()
        B.logra_rowadam_apply(m, B.LOGRA_BF16, S_d, v_new, W_d, lr, float(sc), eps)
        torch.cuda.synchronize()
        dw2 += float(((W_d.double() - W0.double()) ** 2).sum().item())
    realised = 0.5 * phi * dw2
    say("  controller: predicted %.4e, budget %.4e, realised after scaling %.4e" % (kl_pred, delta, realised))
    assert abs(realised / delta - 1) < BF16_TOL


@pytest.mark.parametrize("compute", [B.LOGRA_BF16, B.LOGRA_F32])
def test_sqnorm_batch_equals_single_calls(compute):
    # pass 1 of several matrices in one call == one call per matrix, bit for
    # bit (v', rowsq where requested, sqnorm), shapes from one to many
    # workgroups per matrix and a ragged last workgroup
    dev = device()
    r = 256 if compute == B.LOGRA_BF16 else 40
    shapes = [(520, 1544), (256, 1536), (8200, 136), (1032, 4104), (40, 72)]
    ms, S, v = [], [], []
    for i, (d, k) in enumerate(shapes):
        ms.append(B.MatrixDesc(d, k, r, 3, 5, 20 + i))
        Si, vi, _ = _state(50 + i, d, k, r)
        S.append(Si.to(dev))
        v.append(vi.to(dev))
    v_new_b = [torch.full((m.d,), -1.0, device=dev) for m in ms]
    rowsq_b = [torch.full((m.d,), -1.0, device=dev) if i % 2 == 0 else None for i, m in enumerate(ms)]
    sq_b = torch.full((len(ms),), -1.0, device=dev)
    B.logra_update_sqnorm_batch(ms, compute, S, v, 0.999, 1e-8, v_new_b, sq_b, rowsq_b)
    torch.cuda.synchronize()
    for i, m in enumerate(ms):
        v_new = torch.empty(m.d, device=dev)
        rowsq = torch.empty(m.d, device=dev)
        sq = torch.empty(1, device=dev)
        B.logra_update_sqnorm(m, compute, S[i], v[i], 0.999, 1e-8, v_new, sq, rowsq)
        torch.cuda.synchronize()
        assert torch.equal(v_new, v_new_b[i]), i
        assert torch.equal(sq[0], sq_b[i]), i
        if rowsq_b[i] is not None:
            assert torch.equal(rowsq, rowsq_b[i]), i
