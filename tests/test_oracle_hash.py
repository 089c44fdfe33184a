"""Pins for the oracle's counter hash and sign matrix.

The pages fix only that A is a random-sign r x k matrix with entries
+-1/sqrt(r), redrawn every step and fixed within it ("LoGRA: Scaling LLM
Reinforcement Learning with Low-Rank Gradient Sketches", paragraph "Gradient
sketches."). The generator itself is this library's reading: SplitMix64
keyed by (seed, step, matrix id). Pins: the published SplitMix64 known
answers, the counter layout, bit statistics and E[A^T A] = I.
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_known_answers.txt")


def _known_answers():
    rows = []
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        s, n, v = line.split()
        rows.append((int(s), int(n), int(v)))
    return rows


def test_splitmix64_known_answers():
    rows = _known_answers()
    assert len(rows) == 6
    for seed, n, val in rows:
        assert oracle.splitmix64_output(seed, n) == val


def test_sign_word_is_splitmix64_stream_of_key():
    # Row l = 0 of the sign words is outputs 1, 2, 3, ... of SplitMix64
    # started at the key (counter = ((l << 32) | b) + 1).
    known = {n: v for s, n, v in _known_answers() if s == 1234567}
    for b in range(5):
        assert oracle.sign_word(1234567, 0, b) == known[b + 1]


def test_key_chain_first_stage_matches_known_answer():
    # With seed 0 the first stage of the key is output 1 of SplitMix64(0).
    h0 = oracle.splitmix64_output(0, 1)
    assert h0 == 16294208416658607535
    # key(0, 0, 0) = h(h(h(0) ^ 0) ^ 0): two more first-outputs.
    assert oracle.stream_key(0, 0, 0) == oracle.splitmix64_output(
        oracle.splitmix64_output(h0, 1), 1)


def test_keys_distinct_over_grid():
    keys = {oracle.stream_key(s, t, m) for s in range(4) for t in range(16) for m in range(16)}
    assert len(keys) == 4 * 16 * 16


def _bits(words):
    w = np.asarray(words, dtype=np.uint64)
    return ((w[..., None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(np.int64)


def test_bit_statistics():
    # Many words across (step, matrix): popcount ~ Binomial(64, 1/2) and
    # neighbouring bits (along j and along l) uncorrelated.
    words = np.concatenate([oracle.sign_words(7, step, mid, 64, 640).ravel()
                            for step in range(8) for mid in range(4)])
    bits = _bits(words)                       # (n, 64)
    n = bits.shape[0]
    pc = bits.sum(axis=1)
    z_mean = (pc.mean() - 32.0) / np.sqrt(16.0 / n)
    assert abs(z_mean) < 5
    assert abs(pc.var() / 16.0 - 1.0) < 0.1
    frac = bits.mean()
    assert abs(frac - 0.5) < 5 * np.sqrt(0.25 / bits.size)
    s = 1 - 2 * bits
    corr_j = (s[:, :-1] * s[:, 1:]).mean()
    assert abs(corr_j) < 5 / np.sqrt(s[:, :-1].size)
    W = oracle.sign_words(11, 3, 2, 256, 4096)          # (256, 64)
    S = 1 - 2 * _bits(W)                                  # (256, 64, 64)
    corr_l = (S[:-1] * S[1:]).mean()
    assert abs(corr_l) < 5 / np.sqrt(S[:-1].size)


def test_step_and_matrix_change_about_half_the_signs():
    a = oracle.sign_matrix(0, 0, 5, 64, 1024)
    for other in (oracle.sign_matrix(0, 1, 5, 64, 1024), oracle.sign_matrix(0, 0, 6, 64, 1024),
                  oracle.sign_matrix(1, 0, 5, 64, 1024)):
        same = (np.sign(a) == np.sign(other)).mean()
        assert abs(same - 0.5) < 5 * np.sqrt(0.25 / a.size)


def test_sign_matrix_entries_and_layout():
    r, k = 32, 200   # k not a multiple of 64: last word only partly used
    A = oracle.sign_matrix(3, 4, 9, r, k)
    words = oracle.sign_words(3, 4, 9, r, k)
    assert words.shape == (r, 4)
    c = 1.0 / np.sqrt(r)
    assert np.all(np.abs(A) == c)
    # bit (j mod 64) of word (l, j // 64); bit 1 -> negative
    bits = _bits(words).reshape(r, -1)[:, :k]
    assert np.array_equal(A < 0, bits == 1)
    # diag(A^T A) = r * c^2 = 1 to fp64 rounding
    assert np.allclose(np.einsum("lj,lj->j", A, A), 1.0, rtol=0, atol=1e-14)


def test_expected_AtA_is_identity():
    # E[A^T A] = I: diagonal exactly 1, off-diagonal entries have mean 0 and
    # variance 1/r for iid signs.
    r, k, N = 16, 24, 400
    acc = np.zeros((k, k))
    off_vals = []
    for step in range(N):
        A = oracle.sign_matrix(123, step, 0, r, k)
        M = A.T @ A
        acc += M
        off_vals.append(M[~np.eye(k, dtype=bool)])
    mean = acc / N
    assert np.allclose(np.diag(mean), 1.0, atol=1e-13)
    off = np.concatenate(off_vals)
    off_mean = mean[~np.eye(k, dtype=bool)]
    # each entry of the mean has std sqrt(1/(r N))
    assert np.abs(off_mean).max() < 5 * np.sqrt(1.0 / (r * N))
    assert abs(off.var() * r - 1.0) < 0.05


@pytest.mark.parametrize("r,k", [(1, 1), (16, 64), (32, 65), (256, 3584)])
def test_word_counts(r, k):
    w = oracle.sign_words(0, 0, 0, r, k)
    assert w.shape == (r, (k + 63) // 64)
