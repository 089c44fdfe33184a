"""GPU parity of the two-sided sketch variant (logra_ts_*) through the C ABI
against the oracle (oracle/two_sided.py), on seeded synthetic inputs.

  * projections: the fp32 matrix within 1e-6 of the oracle's fp64 QR factor
    (relative to its largest entry; the fp32 rounding is 6e-8), and the bf16
    operand copy equal, bit for bit and in its layout, to the bf16 rounding of
    the fp32 matrix (zero past the last row);
  * sketches: S_L^T and S_R per row (normwise) within 2e-2 of the oracle's
    fp64 sketches of the same bf16 inputs (the kernels round the projections
    and the projected microbatch to bf16), over several microbatches, ragged
    token counts, every fold plan (tiles split over two token halves, over
    more members, not split), the 7B up projection at its full size, and
    T = 0;
  * update and apply: the moments (a few fp32 roundings of their terms), the
    update G_hat (read out as -W after an apply to W = 0 in fp32) and sqnorm
    against the oracle on the same fp32 state, to 2e-4 + 1e-6 cond(P^T U_R)
    (the coupling's sensitivity to the fp32 rounding of U_R and P); a bf16 W
    to one bf16 rounding plus that tolerance; a padded fp32 W (row stride
    > k, padding untouched);
  * degenerate cases: all-zero state (sqnorm 0, W unchanged bit for bit),
    zero columns of S_R (a singular coupling matrix, truncated on both
    sides), a rank-4 gradient with v held at 1 (G_hat = G / (1 + eps));
  * bitwise repeatability of a whole step.
"""
import numpy as np
import pytest
import torch

from oracle import two_sided as ts
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import BF16_TOL, bf16_w_check, device, f32, rownorm_err, say, to_f64

pytestmark = pytest.mark.gpu

R = 32


def _proj(m, side, dev):
    buf = torch.empty(B.logra_ts_projection_bytes(m, side), dtype=torch.uint8, device=dev)
    B.logra_ts_make_projection(m, side, buf)
    return buf


def _oracle_proj(m, side):
    return ts.projection(m.seed, m.matrix_id, side, m.d if side == 0 else m.k, R)


@pytest.mark.parametrize("n", [32, 520, 4096, 18944])
def test_projection_matches_oracle(n):
    dev = device()
    say("ts projection", n)
    m = B.MatrixDesc(n, n, R, seed=11, matrix_id=n % 7)
    for side in (0, 1):
        buf = _proj(m, side, dev)
        torch.cuda.synchronize()
        P = B.logra_ts_projection_fp32(m, side, buf)
        ref = ts.projection(11, n % 7, side, n, R)
        err = np.abs(to_f64(P) - ref).max() / np.abs(ref).max()
        say("  side %d: max err %.2e" % (side, err))
        assert err < 1e-6
        # the bf16 operand copy: block s of 32 rows, column l, row e
        off = (n * R * 4 + 255) // 256 * 256
        nblk = (n + 31) // 32
        frag = buf[off:off + nblk * 32 * R * 2].view(torch.int16).view(nblk, R, 32).cpu()
        Pp = torch.zeros(nblk * 32, R, dtype=torch.float32)
        Pp[:n] = P.cpu()
        want = Pp.to(torch.bfloat16).view(torch.int16).view(nblk, 32, R).transpose(1, 2)
        bad = (frag != want).nonzero()
        for s_, l_, e_ in bad[:8].tolist():
            x = Pp[32 * s_ + e_, l_]
            say("  mismatch block %d col %d row %d: fp32 %.9e bits %08x gpu %04x want %04x" % (
                s_, l_, e_, float(x), x.view(torch.int32).item() & 0xFFFFFFFF,
                frag[s_, l_, e_].item() & 0xFFFF, want[s_, l_, e_].item() & 0xFFFF))
        assert bad.shape[0] == 0


def _sketch_inputs(T, d, k, n, seed, dev):
    Xs, dYs = [], []
    for i in range(n):
        X, dY = inputs.random_case(seed + 31 * i, T, d, k, dtype=torch.bfloat16, dy_std=1e-2,
                                   outlier_cols=max(1, k // 100))
        Xs.append(X.to(dev))
        dYs.append(dY.to(dev))
    return Xs, dYs


def _sketch_ref(m, Xs, dYs):
    P, Q = _oracle_proj(m, 0), _oracle_proj(m, 1)
    L = Rs = None
    for i, (X, dY) in enumerate(zip(Xs, dYs)):
        L, Rs = ts.sketch_step(to_f64(X), to_f64(dY), P, Q, L, Rs, accumulate=i > 0)
    return L, Rs


def _sketch_run(m, Xs, dYs, pP, pQ, dev):
    T = Xs[0].shape[0]
    ws = torch.empty(max(16, B.logra_ts_sketch_workspace_bytes(m, T)), dtype=torch.uint8, device=dev)
    S_L = torch.full((m.k, R), float("nan"), device=dev)
    S_R = torch.full((m.d, R), float("nan"), device=dev)
    for i, (X, dY) in enumerate(zip(Xs, dYs)):
        B.logra_ts_sketch_accumulate(m, X, dY, pP, pQ, S_L, S_R, i > 0, ws)
    torch.cuda.synchronize()
    return S_L, S_R


SKETCH_CASES = [
    # T, d, k, microbatches; the fold plans they exercise
    (100, 520, 264, 3),      # ragged T, small d and k: several members per tile
    (300, 8200, 136, 2),     # S_R over two token halves per tile, S_L^T over more members
    (1000, 64, 8200, 2),     # the other way round
    (100, 8200, 8200, 2),    # four token steps: one member per tile for both
    (2052, 3592, 1048, 2),   # ragged T over several column chunks of dY
]


@pytest.mark.parametrize("T,d,k,n", SKETCH_CASES)
def test_sketch_matches_oracle(T, d, k, n):
    dev = device()
    say("ts sketch", T, d, k, n)
    m = B.MatrixDesc(d, k, R, seed=5, matrix_id=d + k)
    pP, pQ = _proj(m, 0, dev), _proj(m, 1, dev)
    Xs, dYs = _sketch_inputs(T, d, k, n, 3 * T + d, dev)
    S_L, S_R = _sketch_run(m, Xs, dYs, pP, pQ, dev)
    L, Rs = _sketch_ref(m, Xs, dYs)
    eL, eR = rownorm_err(to_f64(S_L), L.T), rownorm_err(to_f64(S_R), Rs)
    say("  S_L^T %.3e  S_R %.3e" % (eL, eR))
    assert eL < BF16_TOL and eR < BF16_TOL


def test_sketch_at_the_7b_up_shape():
    dev = device()
    T, d, k = 4096, 18944, 3584
    say("ts sketch 7B up", T, d, k)
    wl = inputs.WORKLOADS["qwen7b_up"]
    spec = inputs.MatrixSpec("up", 0, d, k, 5)
    Xs = [inputs.activations(wl, spec, 0, mb, device=dev) for mb in range(2)]
    dYs = [inputs.output_grads(wl, spec, 0, mb, device=dev) for mb in range(2)]
    m = B.MatrixDesc(d, k, R, seed=0, matrix_id=5)
    pP, pQ = _proj(m, 0, dev), _proj(m, 1, dev)
    S_L, S_R = _sketch_run(m, Xs, dYs, pP, pQ, dev)
    L, Rs = _sketch_ref(m, Xs, dYs)
    eL, eR = rownorm_err(to_f64(S_L), L.T), rownorm_err(to_f64(S_R), Rs)
    say("  S_L^T %.3e  S_R %.3e" % (eL, eR))
    assert eL < BF16_TOL and eR < BF16_TOL


def test_sketch_with_no_tokens():
    dev = device()
    m = B.MatrixDesc(520, 264, R, seed=1, matrix_id=1)
    pP, pQ = _proj(m, 0, dev), _proj(m, 1, dev)
    X = torch.empty(0, 264, dtype=torch.bfloat16, device=dev)
    dY = torch.empty(0, 520, dtype=torch.bfloat16, device=dev)
    S_L = torch.full((264, R), 3.0, device=dev)
    S_R = torch.full((520, R), 3.0, device=dev)
    B.logra_ts_sketch_accumulate(m, X, dY, pP, pQ, S_L, S_R, True)
    torch.cuda.synchronize()
    assert bool((S_L == 3).all()) and bool((S_R == 3).all())
    B.logra_ts_sketch_accumulate(m, X, dY, pP, pQ, S_L, S_R, False)
    torch.cuda.synchronize()
    assert bool((S_L == 0).all()) and bool((S_R == 0).all())


# ---------------------------------------------------------------- update --

def _state(d, k, seed, scale=1e-2):
    g = inputs.generator("ts-state", seed, d, k)
    S_L = torch.randn(k, R, generator=g) * scale
    S_R = torch.randn(d, R, generator=g) * scale
    m_L = torch.randn(k, R, generator=g) * scale
    m_R = torch.randn(d, R, generator=g) * scale
    v_L = (0.5 + torch.rand(k, R, generator=g)) * scale * scale
    v_R = (0.5 + torch.rand(d, R, generator=g)) * scale * scale
    return S_L, S_R, m_L, v_L, m_R, v_R


def _run_update(m, st, pP, dev, beta1, beta2, eps, W=None, lr=1.0, scale=1.0):
    """Moments in place on device copies; returns (moments, sqnorm, W after
    apply). W defaults to an fp32 zero matrix, so that -W is G_hat."""
    S_L, S_R, m_L, v_L, m_R, v_R = [t.to(dev) for t in st]
    ws = torch.empty(B.logra_ts_update_workspace_bytes(m), dtype=torch.uint8, device=dev)
    sq = torch.full((1,), float("nan"), device=dev)
    B.logra_ts_update(m, S_L, S_R, pP, m_L, v_L, m_R, v_R, beta1, beta2, eps, sq, ws)
    if W is None:
        W = torch.zeros(m.d, m.k, device=dev)
    B.logra_ts_apply(m, ws, W, lr, scale)
    torch.cuda.synchronize()
    return (m_L, v_L, m_R, v_R), float(sq.item()), W


def _oracle_update(m, st, beta1, beta2, eps):
    S_L, S_R, m_L, v_L, m_R, v_R = [to_f64(t) for t in st]
    P = _oracle_proj(m, 0)
    out = ts.update(S_L.T, S_R, P, m_L.T, v_L.T, m_R, v_R, beta1=f32(beta1), beta2=f32(beta2), eps=f32(eps))
    cond = np.linalg.cond(P.T @ out["U_R"])
    return out, cond


def _moment_errs(st, got, out, beta1, beta2):
    """Error of the fp32 moments over the size of their terms (so that
    cancellation in the first moment does not inflate it)."""
    b1, b2 = f32(beta1), f32(beta2)
    S_L, S_R, m_L, v_L, m_R, v_R = [to_f64(t) for t in st]
    errs = []
    for S, m0, v0, mg, vg, mr, vr in ((S_L, m_L, v_L, got[0], got[1], out["m_L"].T, out["v_L"].T),
                                       (S_R, m_R, v_R, got[2], got[3], out["m_R"], out["v_R"])):
        size_m = np.abs(b1 * m0) + np.abs((1 - b1) * S) + 1e-30
        errs.append(float((np.abs(to_f64(mg) - mr) / size_m).max()))
        errs.append(float((np.abs(to_f64(vg) - vr) / (np.abs(vr) + 1e-30)).max()))
    return max(errs)


UPDATE_CASES = [(520, 264), (4096, 4096), (8200, 136), (18944, 3584)]


@pytest.mark.parametrize("d,k", UPDATE_CASES)
def test_update_matches_oracle(d, k):
    dev = device()
    say("ts update", d, k)
    m = B.MatrixDesc(d, k, R, seed=2, matrix_id=d)
    pP = _proj(m, 0, dev)
    st = _state(d, k, 1)
    beta1, beta2, eps = 0.9, 0.999, 1e-8
    mom, sq, W = _run_update(m, st, pP, dev, beta1, beta2, eps)
    out, cond = _oracle_update(m, st, beta1, beta2, eps)
    e_mom = _moment_errs(st, mom, out, beta1, beta2)
    G_hat = -to_f64(W)
    tol = 2e-4 + 1e-6 * cond
    e_g = rownorm_err(G_hat, out["G_hat"])
    e_sq = abs(sq - out["sqnorm"]) / out["sqnorm"]
    say("  cond %.1f  moments %.2e  G_hat %.2e  sqnorm %.2e  (tol %.1e)" % (cond, e_mom, e_g, e_sq, tol))
    assert e_mom < 4 * 2.0 ** -24
    assert e_g < tol and e_sq < tol


def test_update_applies_to_bf16_and_padded_fp32_w():
    dev = device()
    d, k = 1040, 520
    m = B.MatrixDesc(d, k, R, seed=9, matrix_id=4)
    pP = _proj(m, 0, dev)
    st = _state(d, k, 2)
    beta1, beta2, eps, lr, scale = 0.9, 0.99, 1e-8, 1e-3, 0.5
    out, cond = _oracle_update(m, st, beta1, beta2, eps)
    tol = 2e-4 + 1e-6 * cond
    g = inputs.generator("ts-W", d, k)
    W0 = torch.randn(d, k, generator=g) * 0.02
    # bf16 W
    Wb = W0.to(torch.bfloat16).to(dev)
    _, _, Wb = _run_update(m, st, pP, dev, beta1, beta2, eps, W=Wb, lr=lr, scale=scale)
    W_old = to_f64(W0.to(torch.bfloat16))
    W_ref = W_old - f32(f32(lr) * f32(scale)) * out["G_hat"]
    ok, worst, _ = bf16_w_check(to_f64(Wb), W_ref, W_old, tol=tol)
    say("  bf16 W worst ratio %.3f" % worst)
    assert ok
    # fp32 W inside a wider buffer: row stride k + 24, the padding untouched
    buf = torch.full((d, k + 24), 7.0, device=dev)
    buf[:, :k] = W0.to(dev)
    _, _, _ = _run_update(m, st, pP, dev, beta1, beta2, eps, W=buf[:, :k], lr=lr, scale=scale)
    W_ref = to_f64(W0) - f32(f32(lr) * f32(scale)) * out["G_hat"]
    got = to_f64(buf[:, :k])
    err = rownorm_err(got - to_f64(W0), W_ref - to_f64(W0))
    say("  fp32 W update err %.2e" % err)
    assert err < tol
    assert bool((buf[:, k:] == 7.0).all())


def test_zero_state_gives_zero_update():
    dev = device()
    d, k = 520, 264
    m = B.MatrixDesc(d, k, R, seed=1, matrix_id=2)
    pP = _proj(m, 0, dev)
    st = tuple(torch.zeros(n, R) for n in (k, d, k, k, d, d))
    g = inputs.generator("ts-W0", d, k)
    W = (torch.randn(d, k, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    W0 = W.clone()
    mom, sq, W = _run_update(m, st, pP, dev, 0.9, 0.999, 1e-8, W=W, lr=1e-3)
    assert sq == 0.0
    assert torch.equal(W, W0)
    assert all(bool((t == 0).all()) for t in mom)


def test_singular_coupling_from_zero_columns():
    dev = device()
    d, k = 520, 264
    m = B.MatrixDesc(d, k, R, seed=4, matrix_id=7)
    pP = _proj(m, 0, dev)
    st = list(_state(d, k, 3))
    for i in (1, 4):          # S_R and m_R: columns 5 and 17 zero, so U_R's are
        st[i] = st[i].clone()
        st[i][:, [5, 17]] = 0.0
    st = tuple(st)
    mom, sq, W = _run_update(m, st, pP, dev, 0.9, 0.999, 1e-8)
    out, _ = _oracle_update(m, st, 0.9, 0.999, 1e-8)
    sv = np.linalg.svd(_oracle_proj(m, 0).T @ out["U_R"], compute_uv=False)
    assert sv[-2] <= 1e-12 * sv[0] and sv[-3] > 1e-3 * sv[0]
    kept = sv[sv > 32 * 2.0 ** -23 * sv[0]]
    cond = kept[0] / kept[-1]
    tol = 2e-4 + 1e-6 * cond
    e_g = rownorm_err(-to_f64(W), out["G_hat"])
    e_sq = abs(sq - out["sqnorm"]) / out["sqnorm"]
    say("  rank-30 coupling: G_hat %.2e  sqnorm %.2e  (tol %.1e)" % (e_g, e_sq, tol))
    assert e_g < tol and e_sq < tol


def test_low_rank_gradient_is_recovered():
    # beta1 = 0, beta2 = 1 with v = 1 (U = S / (1 + eps)) and raw sketches of
    # a rank-4 gradient (made by the oracle's projections, stored in fp32):
    # the update is G / (1 + eps)
    dev = device()
    d, k, eps = 1040, 776, 0.25
    m = B.MatrixDesc(d, k, R, seed=8, matrix_id=3)
    pP = _proj(m, 0, dev)
    g = inputs.generator("ts-lowrank", d, k)
    G = (torch.randn(d, 4, generator=g, dtype=torch.float64) @ torch.randn(4, k, generator=g, dtype=torch.float64)).numpy()
    P, Q = _oracle_proj(m, 0), _oracle_proj(m, 1)
    S_L = torch.from_numpy((P.T @ G).T.copy()).float()
    S_R = torch.from_numpy(G @ Q).float()
    st = (S_L, S_R, torch.zeros(k, R), torch.ones(k, R), torch.zeros(d, R), torch.ones(d, R))
    _, sq, W = _run_update(m, st, pP, dev, 0.0, 1.0, eps)
    G_hat = -to_f64(W)
    err = np.abs(G_hat - G / (1 + eps)).max() / np.abs(G).max()
    e_sq = abs(sq - np.sum((G / (1 + eps)) ** 2)) / np.sum((G / (1 + eps)) ** 2)
    say("  rank-4 recovery %.2e  sqnorm %.2e" % (err, e_sq))
    assert err < 1e-4 and e_sq < 1e-4


def test_two_sided_step_is_bitwise_repeatable():
    dev = device()
    T, d, k = 300, 8200, 1040
    m = B.MatrixDesc(d, k, R, seed=3, matrix_id=1)
    Xs, dYs = _sketch_inputs(T, d, k, 2, 77, dev)
    outs = []
    for _ in range(2):
        pP, pQ = _proj(m, 0, dev), _proj(m, 1, dev)
        S_L, S_R = _sketch_run(m, Xs, dYs, pP, pQ, dev)
        st = (S_L, S_R, torch.zeros(k, R), torch.zeros(k, R), torch.zeros(d, R), torch.zeros(d, R))
        mom, sq, W = _run_update(m, st, pP, dev, 0.9, 0.999, 1e-8)
        fp = [B.logra_ts_projection_fp32(m, s, p).clone() for s, p in ((0, pP), (1, pQ))]
        outs.append((fp[0], fp[1], S_L, S_R, mom, sq, W))
    a, b = outs
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)
    assert all(torch.equal(x, y) for x, y in zip(a[4], b[4]))
    assert a[5] == b[5] and torch.equal(a[6], b[6])


def test_sketch_with_strided_activations():
    # X and dY as column slices of wider buffers (row strides k + 40 and
    # d + 24): the same sketches as from contiguous copies, bit for bit, and
    # within the bf16 tolerance of the oracle
    dev = device()
    T, d, k = 300, 1040, 520
    m = B.MatrixDesc(d, k, R, seed=6, matrix_id=2)
    pP, pQ = _proj(m, 0, dev), _proj(m, 1, dev)
    Xs, dYs = _sketch_inputs(T, d, k, 2, 91, dev)
    Xw = [torch.zeros(T, k + 40, dtype=torch.bfloat16, device=dev) for _ in Xs]
    Yw = [torch.zeros(T, d + 24, dtype=torch.bfloat16, device=dev) for _ in dYs]
    for a, b in zip(Xw, Xs):
        a[:, :k] = b
    for a, b in zip(Yw, dYs):
        a[:, :d] = b
    S_L, S_R = _sketch_run(m, [a[:, :k] for a in Xw], [a[:, :d] for a in Yw], pP, pQ, dev)
    S_L2, S_R2 = _sketch_run(m, Xs, dYs, pP, pQ, dev)
    assert torch.equal(S_L, S_L2) and torch.equal(S_R, S_R2)
    L, Rs = _sketch_ref(m, Xs, dYs)
    assert rownorm_err(to_f64(S_L), L.T) < BF16_TOL and rownorm_err(to_f64(S_R), Rs) < BF16_TOL
