"""Pins of the oracle's backward input gradient dX = dY W (the product the
backward pass computes from the same dY the sketch accumulates), against
facts that hold independently of its loops: one-hot gradient rows select
rows of W, an identity W returns dY, an independent library matmul agrees to
fp64 rounding, and the map is linear in dY."""
import numpy as np

import oracle


def test_one_hot_rows_select_rows_of_W():
    rng = np.random.default_rng(1)
    d, k = 13, 29
    W = rng.standard_normal((d, k))
    picks = [0, 5, 12, 7]
    dY = np.zeros((len(picks), d))
    for t, i in enumerate(picks):
        dY[t, i] = 1.0
    assert np.array_equal(oracle.backward_dx_rows(dY, W), W[picks])


def test_identity_W_returns_dY():
    rng = np.random.default_rng(2)
    T, d = 17, 24
    dY = rng.standard_normal((T, d))
    assert np.array_equal(oracle.backward_dx_rows(dY, np.eye(d)), dY)


def test_matches_an_independent_matmul_and_row_subsets():
    rng = np.random.default_rng(3)
    T, d, k = 31, 45, 38
    dY = rng.standard_normal((T, d)) * 1e-2
    W = rng.standard_normal((d, k)) * 0.02
    ref = dY @ W
    got = oracle.backward_dx_rows(dY, W)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    rows = [30, 0, 9]
    assert np.array_equal(oracle.backward_dx_rows(dY, W, rows=rows), got[rows])


def test_linear_in_dY():
    rng = np.random.default_rng(4)
    T, d, k = 9, 20, 11
    a, b = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    W = rng.standard_normal((d, k))
    lhs = oracle.backward_dx_rows(2.0 * a - b, W)
    rhs = 2.0 * oracle.backward_dx_rows(a, W) - oracle.backward_dx_rows(b, W)
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(rhs).max()
