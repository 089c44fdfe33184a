"""GPU parity of the sketch path: logra_sign_words and logra_sketch_accumulate
through the C ABI against the CPU oracle, on the same seeded inputs.

Sign words and indexing are bit-exact. S is compared per row (normwise) at
2e-2 for bf16 inputs and 1e-5 for fp32 inputs. Shapes span several tiles of
every kernel and ragged tails in T, d and k.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import BF16_TOL, F32_TOL, device, rownorm_err, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,step,mid,r,k", [
    (0, 0, 0, 32, 512), (1, 7, 3, 256, 3584), (2**63 + 5, 2**40, 12345, 64, 200),
    (9, 1, 1, 1, 1), (5, 9, 196, 1024, 130)])
def test_sign_words_bit_exact(seed, step, mid, r, k):
    dev = device()
    say("sign_words", seed, step, mid, r, k)
    nb = (k + 63) // 64
    m = B.MatrixDesc(8, k, r, seed, step, mid)
    words = torch.zeros(r * nb, dtype=torch.int64, device=dev)
    B.logra_sign_words(m, words)
    torch.cuda.synchronize()
    got = words.cpu().numpy().view(np.uint64).reshape(r, nb)
    assert np.array_equal(got, oracle.sign_words(seed, step, mid, r, k))


def _run_sketch(m, X_list, dY_list, dev, opts=None):
    S = torch.full((m.d, m.r), float("nan"), dtype=torch.float32, device=dev)
    for n, (X, dY) in enumerate(zip(X_list, dY_list)):
        B.logra_sketch_accumulate(m, X.to(dev), dY.to(dev), S, accumulate=n > 0, opts=opts)
    torch.cuda.synchronize()
    return S


def _ref_sketch(m, X_list, dY_list, rows=None):
    A = oracle.sign_matrix(m.seed, m.step, m.matrix_id, m.r, m.k)
    return oracle.sketch([x.double().numpy() for x in X_list], [y.double().numpy() for y in dY_list],
                         A, rows=rows)


BF16_CASES = [
    # T, d, k, r, microbatches
    (96, 192, 320, 32, 2),
    (300, 136, 520, 64, 3),
    (257, 264, 1000, 128, 2),
    (1000, 520, 1544, 256, 2),
    (130, 72, 72, 256, 1),
    (8, 8, 8, 256, 1),
    (513, 1032, 4104, 256, 1),
    # projections in 64-token workgroups (enough of them to fill the chip),
    # ragged: the last workgroup's second P block lies past the buffer
    (8200, 72, 136, 256, 2),
    (16400, 40, 72, 128, 1),
]


@pytest.mark.parametrize("T,d,k,r,mbs", BF16_CASES)
def test_sketch_bf16_matches_oracle(T, d, k, r, mbs):
    dev = device()
    say("sketch bf16", T, d, k, r, mbs)
    m = B.MatrixDesc(d, k, r, seed=3, step=T, matrix_id=d)
    X_list, dY_list = [], []
    for n in range(mbs):
        X, dY = inputs.random_case(1000 * T + n, T, d, k, dtype=torch.bfloat16, dy_std=1e-2,
                                   outlier_cols=max(1, k // 100))
        X_list.append(X)
        dY_list.append(dY)
    S = _run_sketch(m, X_list, dY_list, dev)
    ref = _ref_sketch(m, X_list, dY_list)
    err = rownorm_err(to_f64(S), ref)
    say("  S rownorm err %.3e" % err)
    assert err < BF16_TOL


# Work splits of the fold: tiles over two token halves that exchange partial
# tiles (d >= 8192 at r = 256, or T r > 2^19), more workgroups than compute
# units (d > 20480), tall tiles over all tokens (fewer than 8 steps of 32, or
# r <= 128 with T r <= 2^19; two epilogue passes), and small d with 8 members
# per tile; ragged T and d throughout.
FOLD_SPLIT_CASES = [
    # T, d, k, r, microbatches
    (300, 8200, 136, 256, 2),
    (4200, 8200, 64, 128, 1),     # T r > 2^19: two token halves at r = 128
    (4096, 512, 64, 256, 2),
    (200, 41000, 72, 32, 2),
    (257, 24008, 64, 64, 2),
    (1000, 9000, 40, 128, 1),
    # small d in tiles of up to 10 blocks, 8 members each (32 x 8 = 256
    # workgroups), one of them ragged in d and T
    (1024, 5120, 64, 32, 2),
    (1000, 5000, 72, 32, 1),
    # small d where taller tiles would not fill the chip: 4-block tiles x 4
    # members (the plan of the 7B stack's q/o/down at 4096 tokens), ragged in d
    (1024, 3584, 64, 32, 1),
    (1000, 3592, 72, 32, 1),
]


@pytest.mark.parametrize("T,d,k,r,mbs", FOLD_SPLIT_CASES)
def test_sketch_bf16_fold_splits(T, d, k, r, mbs):
    dev = device()
    say("sketch bf16 split", T, d, k, r, mbs)
    m = B.MatrixDesc(d, k, r, seed=5, step=T, matrix_id=d)
    X_list, dY_list = [], []
    for n in range(mbs):
        X, dY = inputs.random_case(2000 * T + n, T, d, k, dtype=torch.bfloat16, dy_std=1e-2,
                                   outlier_cols=max(1, k // 100))
        X_list.append(X)
        dY_list.append(dY)
    S = _run_sketch(m, X_list, dY_list, dev)
    ref = _ref_sketch(m, X_list, dY_list)
    err = rownorm_err(to_f64(S), ref)
    say("  S rownorm err %.3e" % err)
    assert err < BF16_TOL


def test_fold_twice_from_one_projection():
    # The fold leaves its sync words zero, so a second fold from the same
    # projection and workspace is valid: it adds the same product again.
    dev = device()
    T, d, k, r = 320, 8208, 96, 256
    m = B.MatrixDesc(d, k, r, 1, 2, 3)
    X, dY = inputs.random_case(77, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    X, dY = X.to(dev), dY.to(dev)
    ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    S = torch.empty(d, r, device=dev)
    B.logra_sketch_project(m, X, ws)
    B.logra_sketch_fold(m, dY, S, False, ws)
    S1 = S.clone()
    B.logra_sketch_fold(m, dY, S, True, ws)
    torch.cuda.synchronize()
    assert torch.equal(S, 2 * S1)   # x + x is exact
    S_acc = torch.empty(d, r, device=dev)
    B.logra_sketch_accumulate(m, X, dY, S_acc, accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(S_acc, S1)


def test_fold_wait_timeout_writes_nan_counts_and_recovers():
    # Forced from the host: with a negative wait limit the two members of
    # every tile give up on each other at once, write their rows as NaN and
    # count themselves in the caller's time-out counter (every kernel still
    # runs to its end). With the default limit, a second fold from the same
    # projection and workspace gives the exact result and counts nothing:
    # the timed-out fold left its sync words usable.
    dev = device()
    T, d, k, r = 320, 8208, 96, 256   # d >= 8192: tiles over two token halves
    say("fold wait time-out", T, d, k, r)
    m = B.MatrixDesc(d, k, r, 1, 2, 3)
    X, dY = inputs.random_case(78, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    X, dY = X.to(dev), dY.to(dev)
    ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    S_ref = torch.empty(d, r, device=dev)
    B.logra_sketch_accumulate(m, X, dY, S_ref, accumulate=False)
    S = torch.zeros(d, r, device=dev)
    timeouts = torch.zeros(1, dtype=torch.int32, device=dev)
    B.logra_sketch_project(m, X, ws)
    B.logra_sketch_fold(m, dY, S, False, ws, opts=B.LaunchOpts(fold_wait_limit=-1, fold_timeouts=timeouts))
    torch.cuda.synchronize()
    assert torch.isnan(S).all()
    # every member of every tile gave up once (128 tiles x 2 members here)
    plan_members = 256
    assert timeouts.item() == plan_members
    timeouts.zero_()
    B.logra_sketch_fold(m, dY, S, False, ws, opts=B.LaunchOpts(fold_timeouts=timeouts))
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref)
    assert timeouts.item() == 0


def test_fold_options_are_per_call():
    # Two folds from one projection, one with a negative wait limit, one with
    # the defaults, launched back to back on two streams: each gets its own
    # setting (no process-wide state), whatever order they run in.
    dev = device()
    T, d, k, r = 320, 8208, 96, 256
    m = B.MatrixDesc(d, k, r, 1, 2, 4)
    X, dY = inputs.random_case(79, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    X, dY = X.to(dev), dY.to(dev)
    S_ref = torch.empty(d, r, device=dev)
    B.logra_sketch_accumulate(m, X, dY, S_ref, accumulate=False)
    ws = [torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    S = [torch.zeros(d, r, device=dev) for _ in range(2)]
    cnt = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(2)]
    streams = [torch.cuda.current_stream(), torch.cuda.Stream(device=dev)]
    streams[1].wait_stream(streams[0])
    for i, lim in enumerate((-1, 0)):
        B.logra_sketch_project(m, X, ws[i], stream=streams[i])
        B.logra_sketch_fold(m, dY, S[i], False, ws[i], stream=streams[i],
                            opts=B.LaunchOpts(fold_wait_limit=lim, fold_timeouts=cnt[i]))
    torch.cuda.synchronize()
    assert torch.isnan(S[0]).all() and cnt[0].item() == 256
    assert torch.equal(S[1], S_ref) and cnt[1].item() == 0


@pytest.mark.parametrize("n", [1, 4])
def test_sketch_concurrency_hint_keeps_parity(n):
    # With a concurrency of 4 the projection of 4040 tokens runs in 64-token
    # workgroups (64 x 2: the last one has a partial P block and one past the
    # buffer), with 1 in 32-token ones; both match the oracle to the same
    # tolerance.
    dev = device()
    T, d, k, r = 4040, 264, 200, 256
    say("sketch concurrency", n, T, d, k, r)
    m = B.MatrixDesc(d, k, r, seed=9, step=n, matrix_id=d)
    X, dY = inputs.random_case(4242 + n, T, d, k, dtype=torch.bfloat16, dy_std=1e-2, outlier_cols=2)
    S = _run_sketch(m, [X], [dY], dev, opts=B.LaunchOpts(sketch_concurrency=n))
    err = rownorm_err(to_f64(S), _ref_sketch(m, [X], [dY]))
    say("  S rownorm err %.3e" % err)
    assert err < BF16_TOL


F32_CASES = [
    (128, 256, 512, 32, 4),     # the tiny fp32 workload's shape
    (77, 45, 130, 20, 2),
    (33, 300, 65, 1, 1),
    (200, 64, 256, 100, 2),
    (5, 3, 1, 7, 3),
]


@pytest.mark.parametrize("T,d,k,r,mbs", F32_CASES)
def test_sketch_f32_matches_oracle(T, d, k, r, mbs):
    dev = device()
    say("sketch f32", T, d, k, r, mbs)
    m = B.MatrixDesc(d, k, r, seed=1, step=2, matrix_id=3)
    X_list, dY_list = [], []
    for n in range(mbs):
        X, dY = inputs.random_case(7 * T + n, T, d, k, dtype=torch.float32, dy_std=1e-3)
        X_list.append(X)
        dY_list.append(dY)
    S = _run_sketch(m, X_list, dY_list, dev)
    ref = _ref_sketch(m, X_list, dY_list)
    # error relative to the magnitude of the summed terms, |dY|^T |X| |A|^T:
    # the fp32 forward-error scale, well defined even where a row cancels
    A = oracle.sign_matrix(m.seed, m.step, m.matrix_id, r, k)
    bound = oracle.sketch([np.abs(x.double().numpy()) for x in X_list],
                          [np.abs(y.double().numpy()) for y in dY_list], np.abs(A))
    got = to_f64(S)
    cond = float((np.abs(got - ref) / np.where(bound > 0, bound, 1.0)).max())
    say("  S err / term magnitude %.3e" % cond)
    assert cond < F32_TOL
    if r >= 16:
        err = rownorm_err(got, ref)
        say("  S rownorm err %.3e" % err)
        assert err < F32_TOL


@pytest.mark.parametrize("r", [64, 256])
def test_one_hot_probe_exposes_signs_exactly(r):
    # X = I (one-hot token rows), dY = I: S = c * Sigma^T exactly (c = 1/sqrt(r)
    # is a power of two here, so bf16 P and fp32 S are exact).
    dev = device()
    n = 264
    say("one-hot probe", n, r)
    m = B.MatrixDesc(n, n, r, seed=77, step=5, matrix_id=9)
    eye = torch.eye(n, dtype=torch.bfloat16)
    S = _run_sketch(m, [eye], [eye], dev)
    A = oracle.sign_matrix(77, 5, 9, r, n)
    assert np.array_equal(to_f64(S), A.T)


def test_accumulate_flag_and_linearity():
    dev = device()
    T, d, k, r = 256, 128, 384, 256
    m = B.MatrixDesc(d, k, r, 0, 1, 2)
    X1, dY1 = inputs.random_case(1, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    X2, dY2 = inputs.random_case(2, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    S12 = _run_sketch(m, [X1, X2], [dY1, dY2], dev)
    S_cat = _run_sketch(m, [torch.cat([X1, X2])], [torch.cat([dY1, dY2])], dev)
    assert rownorm_err(to_f64(S12), to_f64(S_cat)) < BF16_TOL
    # accumulate=0 overwrites whatever S held
    S = torch.randn(d, r, device=dev)
    B.logra_sketch_accumulate(m, X1.to(dev), dY1.to(dev), S, accumulate=False)
    S1 = _run_sketch(m, [X1], [dY1], dev)
    torch.cuda.synchronize()
    assert torch.equal(S, S1)


@pytest.mark.parametrize("T,d,k", [(700, 392, 1032), (600, 8200, 200)])
def test_deterministic_repeat(T, d, k):
    # bitwise repeatable, also where token halves exchange partial tiles and
    # finish in whatever order
    dev = device()
    r = 256
    m = B.MatrixDesc(d, k, r, 4, 4, 4)
    X, dY = inputs.random_case(44, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
    a = _run_sketch(m, [X, X], [dY, dY], dev)
    for _ in range(3):
        b = _run_sketch(m, [X, X], [dY, dY], dev)
        assert torch.equal(a, b)


def test_empty_microbatch_and_zero_gradient():
    dev = device()
    d, k, r = 64, 128, 32
    m = B.MatrixDesc(d, k, r, 0, 0, 0)
    S0 = torch.randn(d, r, device=dev)
    S = S0.clone()
    empty_x = torch.zeros(0, k, dtype=torch.bfloat16, device=dev)
    empty_y = torch.zeros(0, d, dtype=torch.bfloat16, device=dev)
    B.logra_sketch_accumulate(m, empty_x, empty_y, S, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    B.logra_sketch_accumulate(m, empty_x, empty_y, S, accumulate=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0
    S = S0.clone()
    X, _ = inputs.random_case(3, 40, d, k, dtype=torch.bfloat16)
    B.logra_sketch_accumulate(m, X.to(dev), torch.zeros(40, d, dtype=torch.bfloat16, device=dev), S,
                              accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


def test_nan_in_gradient_propagates():
    dev = device()
    T, d, k, r = 64, 64, 128, 32
    m = B.MatrixDesc(d, k, r, 0, 0, 0)
    X, dY = inputs.random_case(5, T, d, k, dtype=torch.bfloat16)
    dY[3, 17] = float("nan")
    S = _run_sketch(m, [X], [dY], dev)
    bad = torch.isnan(S).any(dim=1).cpu()
    assert bad[17].item() and bad.sum().item() == 1


def test_errors_leave_outputs_untouched():
    dev = device()
    T, d, k, r = 64, 64, 128, 32
    m = B.MatrixDesc(d, k, r, 0, 0, 0)
    X, dY = inputs.random_case(5, T, d, k, dtype=torch.bfloat16)
    S0 = torch.randn(d, r, device=dev)
    S = S0.clone()
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(B.LograError) as e:
        B.logra_sketch_accumulate(m, X.to(dev), dY.to(dev), S, accumulate=False, ws=ws)
    assert e.value.status == 3
    bad_m = B.MatrixDesc(d, k, 48, 0, 0, 0)
    with pytest.raises(B.LograError) as e:
        B.logra_sketch_accumulate(bad_m, X.to(dev), dY.to(dev), torch.zeros(d, 48, device=dev), False)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
