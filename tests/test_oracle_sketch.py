"""Pins for the oracle's sketch accumulation S += dY^T (X A^T).

The pages define the sketch as S = G A^T with G the d x k gradient and A the
r x k random matrix, accumulated during backpropagation as microbatches
arrive ("NVIDIA's LoGRA fits RL post-training of a 27B model onto a single
eight-GPU node", sections "What happened" and "Why it matters"; "LoGRA:
Scaling LLM Reinforcement Learning...", paragraph "Gradient sketches.").
Pins: brute force against the dense gradient on tiny shapes, linearity over
microbatches, row independence, the zero-gradient special case, the d x r
state size and the Johnson-Lindenstrauss norm identity.
"""
import os

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(20261202)


def _case(T, d, k, scale=1.0):
    return rng.standard_normal((T, k)), rng.standard_normal((T, d)) * scale


@pytest.mark.parametrize("T,d,k,r", [(1, 1, 1, 1), (3, 5, 7, 4), (17, 9, 70, 16),
                                     (33, 40, 65, 32), (64, 70, 129, 8)])
def test_bruteforce_dense_gradient(T, d, k, r):
    X, dY = _case(T, d, k)
    A = oracle.sign_matrix(1, 2, 3, r, k)
    S = oracle.sketch([X], [dY], A)
    G = dY.T @ X                 # the d x k gradient the method never forms
    S_dense = G @ A.T
    assert S.shape == (d, r)
    assert np.allclose(S, S_dense, rtol=1e-12, atol=1e-12 * np.abs(S_dense).max())


def test_linearity_over_microbatches():
    T, d, k, r = 48, 20, 50, 16
    A = oracle.sign_matrix(0, 7, 1, r, k)
    parts = [_case(T, d, k) for _ in range(3)]
    S_acc = oracle.sketch([p[0] for p in parts], [p[1] for p in parts], A)
    Xc = np.concatenate([p[0] for p in parts])
    dYc = np.concatenate([p[1] for p in parts])
    S_cat = oracle.sketch([Xc], [dYc], A)
    assert np.allclose(S_acc, S_cat, rtol=1e-12, atol=1e-12 * np.abs(S_cat).max())


def test_row_subset_is_exact():
    T, d, k, r = 40, 33, 70, 8
    X, dY = _case(T, d, k)
    A = oracle.sign_matrix(5, 0, 2, r, k)
    full = oracle.sketch([X], [dY], A)
    rows = rng.permutation(d)[:11]
    sub = oracle.sketch([X], [dY], A, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_zero_gradient_leaves_S_unchanged():
    T, d, k, r = 16, 12, 20, 8
    X, _ = _case(T, d, k)
    A = oracle.sign_matrix(0, 0, 0, r, k)
    S0 = rng.standard_normal((d, r))
    P = oracle.project(X, A)
    S1 = oracle.sketch_rows(np.zeros((T, d)), P, S_rows=S0, accumulate=True)
    assert np.array_equal(S1, S0)
    S2 = oracle.sketch_rows(np.zeros((T, d)), P, S_rows=S0, accumulate=False)
    assert np.array_equal(S2, np.zeros_like(S0))


def test_empty_microbatch():
    d, k, r = 6, 10, 4
    A = oracle.sign_matrix(0, 0, 0, r, k)
    P = oracle.project(np.zeros((0, k)), A)
    assert P.shape == (0, r)
    S0 = rng.standard_normal((d, r))
    assert np.array_equal(oracle.sketch_rows(np.zeros((0, d)), P, S_rows=S0, accumulate=True), S0)


def test_projection_bruteforce_and_one_hot():
    # A one-hot row of X exposes one column of A exactly.
    r, k = 16, 40
    A = oracle.sign_matrix(9, 1, 4, r, k)
    X = np.zeros((k, k))
    X[np.arange(k), np.arange(k)] = 1.0
    assert np.array_equal(oracle.project(X, A), A.T)


def test_state_is_d_by_r():
    # The sketch keeps d x r numbers instead of the d x k gradient: k/r fewer.
    d, k, r = 30, 96, 8
    X, dY = _case(5, d, k)
    S = oracle.sketch([X], [dY], oracle.sign_matrix(0, 0, 0, r, k))
    assert S.size == d * r and (d * k) // S.size == k // r


def test_jl_norm_identity_monte_carlo():
    # E ||S_i||^2 = ||G_i||^2 because E[A^T A] = I.
    T, d, k, r, N = 12, 4, 30, 8, 600
    X, dY = _case(T, d, k)
    G = dY.T @ X
    acc = np.zeros(d)
    for step in range(N):
        A = oracle.sign_matrix(42, step, 0, r, k)
        S = oracle.sketch([X], [dY], A)
        acc += (S ** 2).sum(axis=1)
    ratio = (acc / N) / (G ** 2).sum(axis=1)
    # Var ||S_i||^2 / ||G_i||^2 <= 2/r (Gaussian-like bound) -> std of mean
    assert np.all(np.abs(ratio - 1.0) < 5 * np.sqrt(2.0 / (r * N)))


def test_pages_printed_figures_arithmetic():
    vals = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, v = line.split()
            vals[key] = float(v)
    red7 = 100 * (1 - vals["mem_7b_logra_gib"] / vals["mem_7b_dense_gib"])
    red15 = 100 * (1 - vals["mem_1p5b_logra_gib"] / vals["mem_1p5b_dense_gib"])
    assert abs(red7 - vals["mem_7b_reduction_pct"]) < 0.05
    assert abs(red15 - vals["mem_1p5b_reduction_pct"]) < 0.05
    assert abs(100 - vals["mem_7b_reduction_pct"] - vals["remaining_pct_best_case"]) < 1e-9
    # k/r state reduction at the paper's rank for the 7B MLP up projection
    r = int(vals["rank"])
    d, k = 18944, 3584
    assert (d * k) / (d * r) == 14.0


def test_project_matmul_equals_the_loops():
    # The library-matmul form of P = X A^T that the layer-stack tests use
    # gives the plain loops' result up to fp64 rounding, on a ragged shape
    # with outlier columns; and it reproduces the one-hot probe exactly
    # (X = I gives A^T).
    rng = np.random.default_rng(11)
    T, k, r = 37, 203, 24
    X = rng.standard_normal((T, k))
    X[:, [3, 90]] *= 10.0
    A = oracle.sign_matrix(2, 5, 7, r, k)
    P1 = oracle.project(X, A)
    P2 = oracle.project_matmul(X, A)
    assert np.abs(P1 - P2).max() <= 1e-12 * np.abs(P1).max()
    assert np.array_equal(oracle.project_matmul(np.eye(k), A), A.T)
