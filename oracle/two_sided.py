"""CPU oracle of the two-sided sketch variant (TEST INFRASTRUCTURE ONLY: the
test suite, the smoke check and the benchmark's CPU-baseline leg are its only
callers; the HIP library never imports it).

Source: the walk-through page "LoGRA Cuts LLM RL VRAM by 45.7%: Fit 27B on a
Single Node" (eyestech.in), section "Low-Rank Gradient Sketches via Random
Projections". For the
gradient G (d x k here: output rows, input columns) of a linear layer it
keeps two sketches made with fixed, orthonormalized random Gaussian
projections P (d x r) and Q (k x r), r << min(d, k):

    S_L = P^T G   (r x k)      S_R = G Q   (d x r)

summed over the step's microbatches (G = dY^T X per microbatch, so
S_L += (dY P)^T X and S_R += dY^T (X Q)), keeps first and second moments of
both sketches, and rebuilds the update at step time by pseudo-inverse
coupling of the two sketches:

    G_hat = U_R (P^T U_R)^+ U_L,   U = m / (sqrt(v) + eps) per sketch entry,

which for raw sketches of a gradient of rank <= r returns the gradient
itself (the two-sided sketch reconstruction of Tropp, Yurtsever, Udell and
Cevher, 2017). The readings where the page is silent (the generator, the
moment form, where eps goes, what the controller reads) are the library's
and are listed in the design notes; this module follows them step by step in
fp64, with numpy's QR, pinv and matmul as the library primitives.

Gaussian entries: entry (i, j) of the n x r matrix of side s (0: P, the left
projection over d; 1: Q, the right one over k) takes SplitMix64 outputs
c = 2 (i r + j) + 1 and c + 1 of the stream keyed by
stream_key(seed, PROJECTION_STEP + s, matrix_id), u1 = ((w1 >> 11) + 1) 2^-53
in (0, 1], u2 = (w2 >> 11) 2^-53 in [0, 1), and z = sqrt(-2 ln u1) cos(2 pi u2)
(Box and Muller, 1958). The projection is the Q factor of that matrix whose
R factor has a positive diagonal (unique for a full-rank matrix).
"""
from __future__ import annotations

import numpy as np

from . import stream_key

PROJECTION_STEP = 0xFFFFFFFFFFFFFF00   # a step value the sign matrices never take
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64's finaliser on uint64 arrays (wrapping arithmetic)."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def splitmix64_outputs(key: int, counters: np.ndarray) -> np.ndarray:
    """Output number c of the SplitMix64 stream that starts at key, for each c."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(np.uint64(key) + c * _GAMMA)


def projection_key(seed: int, matrix_id: int, side: int) -> int:
    return stream_key(seed, PROJECTION_STEP + side, matrix_id)


def gaussian(seed: int, matrix_id: int, side: int, n: int, r: int) -> np.ndarray:
    """The n x r matrix of standard normal entries of one side."""
    key = projection_key(seed, matrix_id, side)
    idx = np.arange(n * r, dtype=np.uint64)
    w1 = splitmix64_outputs(key, np.uint64(2) * idx + np.uint64(1))
    w2 = splitmix64_outputs(key, np.uint64(2) * idx + np.uint64(2))
    u1 = ((w1 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w2 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return z.reshape(n, r)


def orthonormalize(Z: np.ndarray) -> np.ndarray:
    """Q of Z = Q R with diag(R) > 0."""
    Qf, Rf = np.linalg.qr(np.asarray(Z, dtype=np.float64))
    s = np.sign(np.diag(Rf))
    s[s == 0] = 1.0
    return Qf * s


def projection(seed: int, matrix_id: int, side: int, n: int, r: int) -> np.ndarray:
    """P (side 0, n = d) or Q (side 1, n = k): orthonormal columns."""
    return orthonormalize(gaussian(seed, matrix_id, side, n, r))


def sketch_step(X, dY, P, Q, S_L=None, S_R=None, accumulate=False):
    """One microbatch: S_L (+)= (dY P)^T X (r x k), S_R (+)= dY^T (X Q) (d x r)."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    L = (dY @ P).T @ X
    Rs = dY.T @ (X @ Q)
    if accumulate:
        L = S_L + L
        Rs = S_R + Rs
    return L, Rs


def moments(S, m, v, beta1: float, beta2: float):
    """First and second moments of one sketch, entrywise (no bias correction)."""
    S = np.asarray(S, dtype=np.float64)
    return beta1 * m + (1.0 - beta1) * S, beta2 * v + (1.0 - beta2) * S * S


def normalized(m, v, eps: float):
    return m / (np.sqrt(v) + eps)


# Relative cutoff of the pseudo-inverse per unit of rank: the sketches and
# their moments are fp32 state, so singular values of the coupling matrix at
# most r * eps(fp32) times the largest are below the precision of the data
# (numpy's dtype-aware rule, max(shape) * eps, for fp32 arrays). Where the
# true coupling matrix is singular (a gradient of rank below r) an untruncated
# inverse would be set by that rounding noise.
PINV_RCOND_PER_RANK = float(np.finfo(np.float32).eps)


def coupling(U_R, P):
    """C = (P^T U_R)^+ (r x r) by numpy's SVD pseudo-inverse, singular values
    at most r * eps(fp32) times the largest counted as zero."""
    M = P.T @ U_R
    return np.linalg.pinv(M, rcond=max(M.shape) * PINV_RCOND_PER_RANK)


def reconstruct(U_L, U_R, P):
    """G_hat = U_R (P^T U_R)^+ U_L (d x k)."""
    return U_R @ coupling(U_R, P) @ U_L


def update(S_L, S_R, P, m_L, v_L, m_R, v_R, *, beta1: float, beta2: float, eps: float):
    """The step-time part: moments of both sketches, the normalized sketches,
    the coupling and the rebuilt update with its squared norm."""
    m_L2, v_L2 = moments(S_L, m_L, v_L, beta1, beta2)
    m_R2, v_R2 = moments(S_R, m_R, v_R, beta1, beta2)
    U_L = normalized(m_L2, v_L2, eps)
    U_R = normalized(m_R2, v_R2, eps)
    C = coupling(U_R, P)
    G_hat = U_R @ C @ U_L
    return {"m_L": m_L2, "v_L": v_L2, "m_R": m_R2, "v_R": v_R2, "U_L": U_L, "U_R": U_R, "C": C,
            "G_hat": G_hat, "sqnorm": float(np.sum(G_hat * G_hat))}


def apply(W, G_hat, lr: float, scale: float):
    """W - lr * scale * G_hat."""
    return np.asarray(W, dtype=np.float64) - lr * scale * G_hat
