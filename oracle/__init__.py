"""CPU oracle for LoGRA's sketch-accumulate + RowAdam-apply path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only permitted callers. The product path (the HIP
library and its binding) never imports this package.

The arithmetic of the sketch and the RowAdam step lives in ``oracle.c``
(plain fp64 C, built with gcc). This module only marshals numpy arrays into
it; every array passed in is converted to a C-contiguous float64 (or
int64/uint64) copy first. The host step controller's oracle is plain Python
in ``oracle/controller.py``, and the two-sided sketch variant's (fixed
orthonormal Gaussian projections on both sides, moments of both sketches,
pseudo-inverse coupling) is plain numpy in ``oracle/two_sided.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
    P = ctypes.c_void_p
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_mix64.restype = u64
    lib.oracle_mix64.argtypes = [u64]
    lib.oracle_splitmix64_output.restype = u64
    lib.oracle_splitmix64_output.argtypes = [u64, u64]
    lib.oracle_stream_key.restype = u64
    lib.oracle_stream_key.argtypes = [u64, u64, u64]
    lib.oracle_sign_word.restype = u64
    lib.oracle_sign_word.argtypes = [u64, i64, i64]
    lib.oracle_sign_words.restype = None
    lib.oracle_sign_words.argtypes = [u64, u64, u64, i64, i64, P]
    lib.oracle_sign_matrix.restype = None
    lib.oracle_sign_matrix.argtypes = [u64, u64, u64, i64, i64, P]
    lib.oracle_project.restype = None
    lib.oracle_project.argtypes = [i64, i64, i64, P, i64, P, P]
    lib.oracle_sketch_rows.restype = None
    lib.oracle_sketch_rows.argtypes = [i64, i64, P, i64, P, i64, P, P, ctypes.c_int]
    lib.oracle_reconstruct_rows.restype = None
    lib.oracle_reconstruct_rows.argtypes = [i64, i64, i64, P, P, P]
    lib.oracle_backward_dx_rows.restype = None
    lib.oracle_backward_dx_rows.argtypes = [i64, i64, P, i64, P, i64, i64, P, P]
    lib.oracle_rowadam_rows.restype = dbl
    lib.oracle_rowadam_rows.argtypes = [i64, i64, i64, P, P, P, dbl, dbl, dbl, dbl,
                                        P, P, P, P, P]
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops (timing only)."""
    _load().oracle_set_num_threads(int(n))


# ------------------------------------------------------------------ hash ---

def mix64(z: int) -> int:
    return int(_load().oracle_mix64(z & 0xFFFFFFFFFFFFFFFF))


def splitmix64_output(state: int, n: int) -> int:
    return int(_load().oracle_splitmix64_output(state & 0xFFFFFFFFFFFFFFFF, n))


def stream_key(seed: int, step: int, matrix_id: int) -> int:
    return int(_load().oracle_stream_key(seed, step, matrix_id))


def sign_word(key: int, l: int, b: int) -> int:
    return int(_load().oracle_sign_word(key, l, b))


def sign_words(seed: int, step: int, matrix_id: int, r: int, k: int) -> np.ndarray:
    nb = (k + 63) // 64
    out = np.zeros((r, nb), dtype=np.uint64)
    _load().oracle_sign_words(seed, step, matrix_id, r, k, _ptr(out))
    return out


def sign_matrix(seed: int, step: int, matrix_id: int, r: int, k: int) -> np.ndarray:
    """A (r x k) with entries +-1/sqrt(r)."""
    out = np.zeros((r, k), dtype=np.float64)
    _load().oracle_sign_matrix(seed, step, matrix_id, r, k, _ptr(out))
    return out


# ---------------------------------------------------------------- sketch ---

def project(X, A) -> np.ndarray:
    """P = X A^T (T x r)."""
    X = _f64(X)
    A = _f64(A)
    T, k = X.shape
    r = A.shape[0]
    assert A.shape[1] == k
    P = np.zeros((T, r), dtype=np.float64)
    _load().oracle_project(T, k, r, _ptr(X), k, _ptr(A), _ptr(P))
    return P


def project_matmul(X, A) -> np.ndarray:
    """P = X A^T (T x r) as one fp64 library matmul: the same definition as
    project() (the first factor of S = G A^T = dY^T (X A^T), "NVIDIA's LoGRA
    fits RL post-training of a 27B model onto a single eight-GPU node",
    section "Why it matters"), for the layer-stack tests whose projections
    (up to 8192 x 17408 x 256 per microbatch) the plain loops take minutes
    over. Summation order is the library's; the result agrees with project()
    to fp64 rounding."""
    X = _f64(X)
    A = _f64(A)
    assert A.shape[1] == X.shape[1]
    return np.ascontiguousarray(X @ A.T)


def sketch_rows(dY, P, rows=None, S_rows=None, accumulate=False) -> np.ndarray:
    """S[rows] (+)= dY[:, rows]^T P. Returns the (nrows x r) S rows."""
    dY = _f64(dY)
    P = _f64(P)
    T, d = dY.shape
    r = P.shape[1]
    assert P.shape[0] == T
    if rows is None:
        nrows = d
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.shape[0]
        assert nrows == 0 or (rows_arr.min() >= 0 and rows_arr.max() < d)
    if S_rows is None:
        S_out = np.zeros((nrows, r), dtype=np.float64)
    else:
        S_out = _f64(S_rows).copy()
        assert S_out.shape == (nrows, r)
    _load().oracle_sketch_rows(T, r, _ptr(dY), d, _ptr(P), nrows,
                               None if rows_arr is None else _ptr(rows_arr),
                               _ptr(S_out), 1 if accumulate else 0)
    return S_out


def sketch(X_list, dY_list, A, rows=None) -> np.ndarray:
    """The whole step's sketch: S = sum over microbatches of dY^T (X A^T),
    starting from zero (rows as in sketch_rows)."""
    S = None
    for n, (X, dY) in enumerate(zip(X_list, dY_list)):
        P = project(X, A)
        S = sketch_rows(dY, P, rows=rows, S_rows=S, accumulate=(n > 0))
    return S


def reconstruct_rows(S_rows, A) -> np.ndarray:
    """Ghat rows = S rows A."""
    S_rows = _f64(S_rows)
    A = _f64(A)
    nrows, r = S_rows.shape
    k = A.shape[1]
    assert A.shape[0] == r
    G = np.zeros((nrows, k), dtype=np.float64)
    _load().oracle_reconstruct_rows(k, r, nrows, _ptr(S_rows), _ptr(A), _ptr(G))
    return G


# ----------------------------------------------------------- backward dX ---

def backward_dx_rows(dY, W, rows=None) -> np.ndarray:
    """dX[rows] = dY[rows] W: the input gradient of Y = X W^T for the listed
    token rows (all when rows is None). dY is T x d, W is d x k."""
    dY = _f64(dY)
    W = _f64(W)
    T, d = dY.shape
    assert W.shape[0] == d
    k = W.shape[1]
    if rows is None:
        nrows, rows_arr = T, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.shape[0]
        assert nrows == 0 or (rows_arr.min() >= 0 and rows_arr.max() < T)
    out = np.zeros((nrows, k), dtype=np.float64)
    _load().oracle_backward_dx_rows(d, k, _ptr(dY), d, _ptr(W), k, nrows,
                                    None if rows_arr is None else _ptr(rows_arr), _ptr(out))
    return out


# --------------------------------------------------------------- RowAdam ---

def rowadam_rows(S_rows, A, v, W=None, *, beta2, eps, lr=0.0, scale=1.0):
    """One RowAdam step on the given rows. Returns a dict with rowsq, v_new,
    sqterm (per row), sqnorm (their sum, in row order) and W_new (fp64; None
    when W is None)."""
    S_rows = _f64(S_rows)
    A = _f64(A)
    v = _f64(v)
    nrows, r = S_rows.shape
    k = A.shape[1]
    assert A.shape[0] == r and v.shape == (nrows,)
    rowsq = np.zeros(nrows)
    v_new = np.zeros(nrows)
    sqterm = np.zeros(nrows)
    if W is not None:
        W = _f64(W)
        assert W.shape == (nrows, k)
        W_new = np.zeros((nrows, k))
        wi, wo = _ptr(W), _ptr(W_new)
    else:
        W_new = None
        wi = wo = None
    total = _load().oracle_rowadam_rows(k, r, nrows, _ptr(S_rows), _ptr(A), _ptr(v),
                                        float(beta2), float(eps), float(lr), float(scale),
                                        wi, wo, _ptr(rowsq), _ptr(v_new), _ptr(sqterm))
    return {"rowsq": rowsq, "v_new": v_new, "sqterm": sqterm,
            "sqnorm": float(total), "W_new": W_new}
