"""Predicted-KL step controller: the C-ABI host function against its oracle,
and the oracle pinned to the RowAdam update it predicts (no GPU needed).

The controller's readings are stated in include/logra.h next to
logra_kl_step_scale: isotropic Fisher phi I, so KL(dW) = 1/2 phi ||dW||^2,
one shrink factor per step, a linearly annealed budget.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import controller as oc


@pytest.fixture(scope="module")
def B():
    from rank_gradient_sketching_sketch_amd import binding
    binding.load_library()
    return binding


def _ghat_case(seed, d, k, r):
    rng = np.random.default_rng(seed)
    A = oracle.sign_matrix(seed, 3, 7, r, k)
    S = rng.normal(size=(d, r)) * 1e-2
    v = rng.uniform(1e-8, 1e-6, size=d)
    W = rng.normal(size=(d, k)) * 0.02
    return S, A, v, W


def test_predicted_kl_is_half_phi_norm_of_the_update():
    # Pin: the prediction from the sketch's sqnorms equals 1/2 phi ||dW||^2 of
    # the RowAdam update the oracle actually applies (W_new - W), summed over
    # matrices; a dropped lr^2, the 1/2 or a wrong sqnorm definition fails it.
    lr, phi, beta2, eps = 3e-3, 0.7, 0.999, 1e-8
    sq, dw2 = [], 0.0
    for m, (d, k, r) in enumerate([(24, 40, 8), (16, 72, 16), (8, 64, 32)]):
        S, A, v, W = _ghat_case(10 + m, d, k, r)
        ref = oracle.rowadam_rows(S, A, v, W, beta2=beta2, eps=eps, lr=lr, scale=1.0)
        sq.append(ref["sqnorm"])
        dw2 += float(np.sum((ref["W_new"] - W) ** 2))
    assert math.isclose(oc.predicted_kl(sq, lr, phi), 0.5 * phi * dw2, rel_tol=1e-10)


def test_scaled_update_meets_the_budget():
    # Pin: applying the controller's gamma as RowAdam's scale gives an update
    # whose 1/2 phi ||dW||^2 is exactly the budget when it binds, and the
    # unscaled prediction when it does not (quadratic model, closed form).
    lr, phi, beta2, eps = 1e-2, 2.0, 0.9, 1e-8
    S, A, v, W = _ghat_case(3, 32, 96, 16)
    full = oracle.rowadam_rows(S, A, v, W, beta2=beta2, eps=eps, lr=lr, scale=1.0)
    kl_full = 0.5 * phi * float(np.sum((full["W_new"] - W) ** 2))
    for delta, binds in [(0.25 * kl_full, True), (4.0 * kl_full, False)]:
        scales, kl, kl_after = oc.step_scale([full["sqnorm"]], lr, phi, delta)
        assert math.isclose(kl, kl_full, rel_tol=1e-10)
        out = oracle.rowadam_rows(S, A, v, W, beta2=beta2, eps=eps, lr=lr, scale=scales[0])
        kl_scaled = 0.5 * phi * float(np.sum((out["W_new"] - W) ** 2))
        assert math.isclose(kl_scaled, delta if binds else kl_full, rel_tol=1e-9)
        assert math.isclose(kl_after, kl_scaled, rel_tol=1e-9)
        assert (scales[0] < 1.0) == binds


def test_budget_anneal_endpoints_and_shape():
    assert oc.kl_budget(0, 0.1, 0.02, 100) == 0.1
    assert oc.kl_budget(100, 0.1, 0.02, 100) == 0.02
    assert oc.kl_budget(5000, 0.1, 0.02, 100) == 0.02
    assert math.isclose(oc.kl_budget(25, 0.1, 0.02, 100), 0.08, rel_tol=1e-15)
    assert oc.kl_budget(7, 0.1, 0.02, 0) == 0.02
    vals = [oc.kl_budget(t, 0.1, 0.02, 100) for t in range(120)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def test_c_abi_matches_oracle(B):
    rng = np.random.default_rng(5)
    for trial in range(50):
        n = int(rng.integers(1, 500))
        q = (rng.lognormal(mean=0.0, sigma=3.0, size=n)).astype(np.float32)
        lr = float(np.float32(10.0 ** rng.uniform(-7, -2)))
        phi = float(10.0 ** rng.uniform(-2, 2))
        kl0 = oc.predicted_kl(q, lr, phi)
        delta = float(kl0 * 10.0 ** rng.uniform(-2, 1))
        s_c, kl_c, after_c = B.logra_kl_step_scale(q, lr, phi, delta)
        s_o, kl_o, after_o = oc.step_scale([float(x) for x in q], lr, phi, delta)
        assert math.isclose(kl_c, kl_o, rel_tol=1e-12)
        assert math.isclose(after_c, after_o, rel_tol=1e-12)
        np.testing.assert_allclose(s_c, np.float32(s_o), rtol=1e-7)
    budget = B.KLBudget(0.1, 0.02, 100)
    for t in [0, 1, 37, 99, 100, 101, 10 ** 12]:
        assert math.isclose(B.logra_kl_budget_at(budget, t), oc.kl_budget(t, 0.1, 0.02, 100), rel_tol=1e-15)


def test_c_abi_special_cases(B):
    # under budget: gamma = 1; zero budget with a nonzero update: gamma = 0
    lr = float(np.float32(0.1))   # the value the C ABI receives
    s, kl, after = B.logra_kl_step_scale([1.0, 2.0], lr, 1.0, 1.0)
    assert np.all(s == 1.0) and math.isclose(kl, 0.5 * lr * lr * 3.0, rel_tol=1e-15) and after == kl
    s, kl, after = B.logra_kl_step_scale([1.0, 2.0], 0.1, 1.0, 0.0)
    assert np.all(s == 0.0) and after == 0.0
    # an empty update stays unscaled even with a zero budget
    s, kl, after = B.logra_kl_step_scale([0.0, 0.0], 0.1, 1.0, 0.0)
    assert np.all(s == 1.0) and kl == 0.0
    # non-finite or negative sqnorm: that matrix is skipped and left out
    s, kl, _ = B.logra_kl_step_scale([4.0, float("nan"), float("inf"), -1.0, 4.0], 1.0, 1.0, 1.0)
    assert s[1] == 0.0 and s[2] == 0.0 and s[3] == 0.0
    assert math.isclose(kl, 4.0) and math.isclose(s[0], 0.5) and s[0] == s[4]
    # homogeneity: sqnorm x alpha^2 -> gamma / alpha while the budget binds
    s1, _, _ = B.logra_kl_step_scale([8.0, 2.0], 1.0, 1.0, 0.5)
    s2, _, _ = B.logra_kl_step_scale([32.0, 8.0], 1.0, 1.0, 0.5)
    assert math.isclose(float(s2[0]), float(s1[0]) / 2.0, rel_tol=1e-6)


def test_c_abi_rejects_bad_arguments(B):
    from rank_gradient_sketching_sketch_amd.binding import LograError
    for args in [([1.0], 0.1, 0.0, 1.0), ([1.0], 0.1, -1.0, 1.0), ([1.0], 0.1, 1.0, -1.0),
                 ([1.0], float("nan"), 1.0, 1.0), ([1.0], 0.1, 1.0, float("inf"))]:
        with pytest.raises(LograError):
            B.logra_kl_step_scale(*args)
    assert math.isnan(B.logra_kl_budget_at(B.KLBudget(-1.0, 0.1, 10), 3))
