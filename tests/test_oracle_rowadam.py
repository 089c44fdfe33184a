"""Pins for the oracle's reconstruction Ghat = S A and RowAdam step.

The pages: the full-size estimate S A exists only when the update is applied
("NVIDIA's LoGRA fits RL post-training...", section "Why it matters");
RowAdam keeps running estimates of squared row magnitudes and no first moment
(same page, "What happened" and "Why it matters"); the step controller reads
a prediction computed from the sketch before each update ("LoGRA: Scaling
LLM Reinforcement Learning...", paragraph "Step control."). Pins: brute force
Ghat = G A^T A; unbiasedness and the closed-form error E||Ghat - G||^2 =
((k-1)/r)||G||^2; k = 1 reduces exactly to torch.optim.RMSprop; beta2, scale
and eps special cases; row normalisation; row permutation equivariance.
"""
import numpy as np
import pytest
import torch

import oracle

rng = np.random.default_rng(7)


def _G(d, k):
    return rng.standard_normal((d, k))


def test_reconstruction_bruteforce():
    d, k, r = 9, 50, 16
    G = _G(d, k)
    A = oracle.sign_matrix(2, 3, 4, r, k)
    S = G @ A.T
    Gh = oracle.reconstruct_rows(S, A)
    assert np.allclose(Gh, G @ A.T @ A, rtol=1e-12, atol=1e-12)
    assert np.allclose(Gh, S @ A, rtol=1e-12, atol=1e-12)


def test_reconstruction_unbiased_and_closed_form_error():
    d, k, r, N = 3, 40, 8, 2000
    G = _G(d, k)
    mean = np.zeros_like(G)
    err2 = 0.0
    rowsq = np.zeros(d)
    for step in range(N):
        A = oracle.sign_matrix(77, step, 1, r, k)
        Gh = oracle.reconstruct_rows(G @ A.T, A)
        mean += Gh
        err2 += ((Gh - G) ** 2).sum()
        rowsq += oracle.rowadam_rows(G @ A.T, A, np.zeros(d), beta2=0.5, eps=0.0)["rowsq"]
    mean /= N
    g2 = (G ** 2).sum()
    # normwise error of the N-sample mean is about sqrt((k-1)/(r N))
    assert np.sqrt(((mean - G) ** 2).sum() / g2) < 3 * np.sqrt((k - 1) / (r * N))
    ratio = (err2 / N) / g2
    assert abs(ratio / ((k - 1) / r) - 1.0) < 0.08
    # E[rowsq_i] = (1 + (k-1)/r) ||G_i||^2
    ex = (1 + (k - 1) / r) * (G ** 2).sum(axis=1)
    assert np.all(np.abs(rowsq / N / ex - 1.0) < 0.15)


def test_k_equals_one_is_rmsprop():
    # With k = 1, A^T A = 1 exactly, so Ghat = G and RowAdam is RMSprop with
    # alpha = beta2, no momentum, not centred, eps outside the sqrt.
    d, r, steps = 6, 16, 4
    lr, scale, beta2, eps = 1e-2, 0.7, 0.9, 1e-8
    W0 = rng.standard_normal((d, 1))
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float64))
    opt = torch.optim.RMSprop([p], lr=lr * scale, alpha=beta2, eps=eps, momentum=0.0,
                              centered=False, weight_decay=0.0)
    W = W0.copy()
    v = np.zeros(d)
    for step in range(steps):
        T = 5
        X = rng.standard_normal((T, 1))
        dY = rng.standard_normal((T, d))
        G = dY.T @ X
        A = oracle.sign_matrix(0, step, 0, r, 1)
        S = oracle.sketch([X], [dY], A)
        out = oracle.rowadam_rows(S, A, v, W, beta2=beta2, eps=eps, lr=lr, scale=scale)
        W, v = out["W_new"], out["v_new"]
        p.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
        assert np.allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-14)
        assert np.allclose(v, opt.state[p]["square_avg"].numpy().ravel(), rtol=1e-12, atol=0)


def test_beta2_and_scale_special_cases():
    d, k, r = 7, 33, 8
    A = oracle.sign_matrix(0, 1, 2, r, k)
    S = rng.standard_normal((d, r))
    v = rng.uniform(1e-3, 1e-2, d)
    W = rng.standard_normal((d, k))
    o0 = oracle.rowadam_rows(S, A, v, W, beta2=0.0, eps=1e-8, lr=1e-3, scale=1.0)
    assert np.allclose(o0["v_new"], o0["rowsq"] / k, rtol=1e-15, atol=0)
    o1 = oracle.rowadam_rows(S, A, v, W, beta2=1.0, eps=1e-8, lr=1e-3, scale=1.0)
    assert np.array_equal(o1["v_new"], v)
    os_ = oracle.rowadam_rows(S, A, v, W, beta2=0.9, eps=1e-8, lr=1e-3, scale=0.0)
    assert np.array_equal(os_["W_new"], W)


def test_row_normalisation_closed_form():
    # v = 0, beta2 = 0, eps = 0: v'_i = ||Ghat_i||^2 / k, so every row of the
    # update has RMS exactly lr*scale and sqnorm = d * k.
    d, k, r = 5, 64, 16
    A = oracle.sign_matrix(3, 0, 0, r, k)
    S = rng.standard_normal((d, r))
    W = rng.standard_normal((d, k))
    lr, scale = 1e-2, 0.5
    o = oracle.rowadam_rows(S, A, np.zeros(d), W, beta2=0.0, eps=0.0, lr=lr, scale=scale)
    dW = o["W_new"] - W
    assert np.allclose((dW ** 2).mean(axis=1), (lr * scale) ** 2, rtol=1e-10)
    assert abs(o["sqnorm"] - d * k) < 1e-9 * d * k
    # the update points against Ghat
    Gh = oracle.reconstruct_rows(S, A)
    assert np.all((dW * Gh) <= 0)


def test_sqnorm_equals_rowsq_weighted_sum():
    # sqnorm is computed literally; it must equal sum_i rowsq_i u_i^2.
    d, k, r = 11, 70, 16
    A = oracle.sign_matrix(5, 5, 5, r, k)
    S = rng.standard_normal((d, r)) * 1e-2
    v = rng.uniform(1e-6, 1e-4, d)
    eps = 1e-3
    o = oracle.rowadam_rows(S, A, v, beta2=0.99, eps=eps)
    u = 1.0 / (np.sqrt(o["v_new"]) + eps)
    assert np.isclose(o["sqnorm"], (o["rowsq"] * u ** 2).sum(), rtol=1e-12)
    assert np.allclose(o["sqterm"], o["rowsq"] * u ** 2, rtol=1e-12)


def test_homogeneity():
    d, k, r = 4, 40, 8
    A = oracle.sign_matrix(0, 0, 0, r, k)
    S = rng.standard_normal((d, r))
    a = oracle.rowadam_rows(S, A, np.ones(d), beta2=0.5, eps=1e-8)
    b = oracle.rowadam_rows(3.0 * S, A, np.ones(d), beta2=0.5, eps=1e-8)
    assert np.allclose(b["rowsq"], 9.0 * a["rowsq"], rtol=1e-12)


def test_row_permutation_equivariance():
    d, k, r = 13, 45, 8
    A = oracle.sign_matrix(8, 1, 3, r, k)
    S = rng.standard_normal((d, r))
    v = rng.uniform(0, 1e-3, d)
    W = rng.standard_normal((d, k))
    perm = rng.permutation(d)
    a = oracle.rowadam_rows(S, A, v, W, beta2=0.9, eps=1e-8, lr=0.1, scale=0.9)
    b = oracle.rowadam_rows(S[perm], A, v[perm], W[perm], beta2=0.9, eps=1e-8, lr=0.1, scale=0.9)
    for key in ("rowsq", "v_new", "sqterm"):
        assert np.array_equal(b[key], a[key][perm])
    assert np.array_equal(b["W_new"], a["W_new"][perm])


@pytest.mark.parametrize("eps", [1e-8, 1e-2])
def test_eps_outside_sqrt(eps):
    # u = 1/(sqrt(v') + eps): check against v' from beta2 = 0 (v' = rowsq/k)
    d, k, r = 3, 16, 4
    A = oracle.sign_matrix(1, 1, 1, r, k)
    S = rng.standard_normal((d, r))
    W = np.zeros((d, k))
    o = oracle.rowadam_rows(S, A, np.zeros(d), W, beta2=0.0, eps=eps, lr=1.0, scale=1.0)
    Gh = oracle.reconstruct_rows(S, A)
    rms = np.sqrt((Gh ** 2).mean(axis=1))
    assert np.allclose(-o["W_new"], Gh / (rms + eps)[:, None], rtol=1e-12)
