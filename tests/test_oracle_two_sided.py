"""Pins of the two-sided sketch oracle (oracle/two_sided.py) against what the
walk-through page "LoGRA Cuts LLM RL VRAM by 45.7%: Fit 27B on a Single Node"
(section "Low-Rank Gradient Sketches via Random Projections") and the
mathematics fix, none of them a retyped formula:

  * its SplitMix64 stream equals the C oracle's (pinned by the published
    known answers in tests/golden/), on many keys and counters;
  * the Gaussian entries pass a Kolmogorov-Smirnov test against the normal
    law and have its mean, variance and fourth moment;
  * the projections have orthonormal columns and span the Gaussian matrix
    with a positive-diagonal triangular factor (the unique QR);
  * the sketches equal P^T G and G Q of the explicit gradient (plain loops on
    tiny inputs) and add over microbatches;
  * the pseudo-inverse coupling returns a gradient of rank <= r exactly from
    its raw sketches (the two-sided sketch identity), and satisfies the four
    Moore-Penrose conditions, also for a singular coupling matrix;
  * the moments reduce to the sketch and its square for beta = 0 and stay put
    for beta = 1; the full update reduces to the exact gradient / (1 + eps)
    when the second moment is held at one;
  * the update's squared norm equals the trace form of the two Gram matrices.
"""
import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import two_sided as ts


def test_splitmix_stream_matches_the_c_oracle():
    rng = np.random.default_rng(0)
    keys = [0, 1, 2**63 + 5, int(rng.integers(0, 2**63)) * 2 + 1]
    counters = np.array([1, 2, 3, 1000, 2**40 + 7, 2**63 - 1], dtype=np.uint64)
    for key in keys:
        got = ts.splitmix64_outputs(key, counters)
        want = [oracle.splitmix64_output(key, int(c)) for c in counters]
        assert [int(x) for x in got] == want


def test_gaussian_entries_follow_the_normal_law():
    Z = ts.gaussian(7, 3, 0, 4096, 32).ravel()
    n = Z.size
    assert abs(Z.mean()) < 5 / np.sqrt(n)
    assert abs(Z.var() - 1) < 5 * np.sqrt(2 / n)
    assert abs(np.mean(Z ** 4) - 3) < 5 * np.sqrt(96 / n)
    assert scipy.stats.kstest(Z, "norm").pvalue > 1e-4
    # the two sides and two matrices are different streams
    assert not np.allclose(ts.gaussian(7, 3, 1, 64, 32), ts.gaussian(7, 3, 0, 64, 32))
    assert not np.allclose(ts.gaussian(7, 4, 0, 64, 32), ts.gaussian(7, 3, 0, 64, 32))
    # entry (i, j) depends on (i, j) only, not on n
    assert np.array_equal(ts.gaussian(7, 3, 0, 64, 32), ts.gaussian(7, 3, 0, 128, 32)[:64])


@pytest.mark.parametrize("n,r", [(64, 16), (520, 32), (4096, 32)])
def test_projection_is_the_unique_qr_factor(n, r):
    Z = ts.gaussian(1, 2, 1, n, r)
    P = ts.projection(1, 2, 1, n, r)
    assert np.abs(P.T @ P - np.eye(r)).max() < 1e-12
    R = P.T @ Z
    assert np.abs(np.tril(R, -1)).max() < 1e-10 * np.abs(R).max()
    assert (np.diag(R) > 0).all()
    assert np.abs(P @ R - Z).max() < 1e-10 * np.abs(Z).max()


def test_sketches_equal_the_projected_explicit_gradient():
    rng = np.random.default_rng(3)
    T, d, k, r = 5, 7, 6, 3
    P = ts.orthonormalize(rng.standard_normal((d, r)))
    Q = ts.orthonormalize(rng.standard_normal((k, r)))
    X1, dY1 = rng.standard_normal((T, k)), rng.standard_normal((T, d))
    X2, dY2 = rng.standard_normal((T, k)), rng.standard_normal((T, d))
    G = np.zeros((d, k))
    for X, dY in ((X1, dY1), (X2, dY2)):
        for t in range(T):
            for i in range(d):
                for j in range(k):
                    G[i, j] += dY[t, i] * X[t, j]
    SL = np.zeros((r, k))
    SR = np.zeros((d, r))
    for a in range(r):
        for j in range(k):
            SL[a, j] = sum(P[i, a] * G[i, j] for i in range(d))
    for i in range(d):
        for a in range(r):
            SR[i, a] = sum(G[i, j] * Q[j, a] for j in range(k))
    L1, R1 = ts.sketch_step(X1, dY1, P, Q)
    L, Rs = ts.sketch_step(X2, dY2, P, Q, L1, R1, accumulate=True)
    assert np.abs(L - SL).max() < 1e-12 * np.abs(SL).max()
    assert np.abs(Rs - SR).max() < 1e-12 * np.abs(SR).max()
    L2, R2 = ts.sketch_step(X2, dY2, P, Q)
    assert np.allclose(L, L1 + L2, rtol=0, atol=1e-13) and np.allclose(Rs, R1 + R2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("rank", [1, 5, 16])
def test_coupling_recovers_a_low_rank_gradient_exactly(rank):
    rng = np.random.default_rng(rank)
    d, k, r = 96, 80, 16
    G = rng.standard_normal((d, rank)) @ rng.standard_normal((rank, k))
    P = ts.projection(0, 1, 0, d, r)
    Q = ts.projection(0, 1, 1, k, r)
    S_L, S_R = P.T @ G, G @ Q
    G_hat = ts.reconstruct(S_L, S_R, P)
    assert np.abs(G_hat - G).max() < 1e-9 * np.abs(G).max()


def test_coupling_is_the_moore_penrose_inverse():
    rng = np.random.default_rng(9)
    d, r = 64, 8
    P = ts.projection(2, 2, 0, d, r)
    for U_R in (rng.standard_normal((d, r)),
                rng.standard_normal((d, 3)) @ rng.standard_normal((3, r)),   # rank 3: singular coupling
                np.zeros((d, r))):
        M = P.T @ U_R
        C = ts.coupling(U_R, P)
        tol = 1e-10 * max(1.0, np.abs(M).max() * np.abs(C).max())
        assert np.abs(M @ C @ M - M).max() <= tol * max(1.0, np.abs(M).max())
        assert np.abs(C @ M @ C - C).max() <= tol * max(1.0, np.abs(C).max())
        assert np.abs((M @ C).T - M @ C).max() <= tol
        assert np.abs((C @ M).T - C @ M).max() <= tol


def test_moments_special_cases():
    rng = np.random.default_rng(4)
    S = rng.standard_normal((5, 6))
    m0, v0 = rng.standard_normal((5, 6)), rng.random((5, 6))
    m, v = ts.moments(S, m0, v0, 0.0, 0.0)
    assert np.array_equal(m, S) and np.array_equal(v, S * S)
    m, v = ts.moments(S, m0, v0, 1.0, 1.0)
    assert np.array_equal(m, m0) and np.array_equal(v, v0)
    # two steps by hand: m2 = b1 (b1 m0 + (1 - b1) S1) + (1 - b1) S2
    S2 = rng.standard_normal((5, 6))
    b1, b2 = 0.9, 0.99
    m1, v1 = ts.moments(S, m0, v0, b1, b2)
    m2, v2 = ts.moments(S2, m1, v1, b1, b2)
    assert np.allclose(m2, b1 * b1 * m0 + b1 * (1 - b1) * S + (1 - b1) * S2, rtol=1e-14, atol=0)
    assert np.allclose(v2, b2 * b2 * v0 + b2 * (1 - b2) * S * S + (1 - b2) * S2 * S2, rtol=1e-14, atol=0)


def test_update_reduces_to_the_gradient_when_the_second_moment_is_one():
    # beta1 = 0 (m = the sketch), beta2 = 1 with v = 1 (v stays 1): U = S / (1 + eps),
    # and the coupling scales inversely with U_R, so G_hat = G / (1 + eps) for a
    # gradient of rank <= r
    rng = np.random.default_rng(6)
    d, k, r, eps = 72, 64, 16, 0.25
    G = rng.standard_normal((d, 4)) @ rng.standard_normal((4, k))
    P = ts.projection(5, 5, 0, d, r)
    Q = ts.projection(5, 5, 1, k, r)
    S_L, S_R = P.T @ G, G @ Q
    out = ts.update(S_L, S_R, P, np.zeros_like(S_L), np.ones_like(S_L), np.zeros_like(S_R), np.ones_like(S_R),
                    beta1=0.0, beta2=1.0, eps=eps)
    assert np.abs(out["G_hat"] - G / (1 + eps)).max() < 1e-9 * np.abs(G).max()
    W = rng.standard_normal((d, k))
    assert np.array_equal(ts.apply(W, out["G_hat"], 0.0, 1.0), W)


def test_sqnorm_equals_the_gram_trace_form():
    rng = np.random.default_rng(8)
    d, k, r = 40, 36, 8
    P = ts.projection(3, 1, 0, d, r)
    S_L, S_R = rng.standard_normal((r, k)), rng.standard_normal((d, r))
    out = ts.update(S_L, S_R, P, rng.standard_normal((r, k)), rng.random((r, k)), rng.standard_normal((d, r)),
                    rng.random((d, r)), beta1=0.9, beta2=0.99, eps=1e-8)
    C, U_L, U_R = out["C"], out["U_L"], out["U_R"]
    trace_form = float(np.sum((C.T @ (U_R.T @ U_R) @ C) * (U_L @ U_L.T)))
    assert abs(out["sqnorm"] - trace_form) < 1e-10 * abs(trace_form)


def test_coupling_truncates_at_the_fp32_precision_of_the_data():
    # U_R = P M0 with P orthonormal gives the coupling matrix M0 itself; with
    # singular values 1, 1e-3, 1e-5, 1e-7 (r = 4: cutoff 4 * 2^-23 = 4.8e-7)
    # the pseudo-inverse keeps the first three and drops the last, in closed
    # form V diag(1, 1e3, 1e5, 0) U^T
    rng = np.random.default_rng(12)
    r = 4
    Uo = ts.orthonormalize(rng.standard_normal((r, r)))
    Vo = ts.orthonormalize(rng.standard_normal((r, r)))
    s = np.array([1.0, 1e-3, 1e-5, 1e-7])
    M0 = Uo @ np.diag(s) @ Vo.T
    P = ts.projection(4, 4, 0, 40, r)
    C = ts.coupling(P @ M0, P)
    want = Vo @ np.diag([1.0, 1e3, 1e5, 0.0]) @ Uo.T
    assert np.abs(C - want).max() < 1e-6 * np.abs(want).max()


def test_low_rank_recovery_under_fp32_rounding_of_the_sketches():
    # sketches of a rank-4 gradient stored in fp32: the truncated coupling
    # drops the 28 directions where the coupling matrix holds rounding noise
    # only (its norm is 1 / sigma_4, not 1 / (noise)), and returns the
    # gradient to fp32 accuracy
    rng = np.random.default_rng(13)
    d, k, r = 200, 160, 32
    G = rng.standard_normal((d, 4)) @ rng.standard_normal((4, k))
    P = ts.projection(6, 1, 0, d, r)
    Q = ts.projection(6, 1, 1, k, r)
    S_L = (P.T @ G).astype(np.float32).astype(np.float64)
    S_R = (G @ Q).astype(np.float32).astype(np.float64)
    sv = np.linalg.svd(P.T @ S_R, compute_uv=False)
    assert sv[4] < 1e-7 * sv[0] < sv[3]
    C = ts.coupling(S_R, P)
    assert abs(np.linalg.norm(C, 2) - 1 / sv[3]) < 1e-6 / sv[3]
    G_hat = ts.reconstruct(S_L, S_R, P)
    assert np.abs(G_hat - G).max() < 1e-6 * np.abs(G).max()
