"""ctypes binding of liblogra.so (declared in include/logra.h).

Argument marshalling only: tensors become device pointers, leading
dimensions and dtypes are read from the tensors, the stream defaults to
torch's current stream. Every step of the computation runs in the HIP
kernels behind the C ABI; there is no fallback of any kind, and a missing or
unloadable library raises LograError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblogra.so")

LOGRA_F32 = 0
LOGRA_BF16 = 1
_STATUS = {0: "LOGRA_OK", 1: "LOGRA_ERR_INVALID_ARGUMENT", 2: "LOGRA_ERR_UNSUPPORTED",
           3: "LOGRA_ERR_WORKSPACE", 4: "LOGRA_ERR_HIP"}


class LograError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, _STATUS.get(status, str(status))))


class MatrixDesc(ctypes.Structure):
    """logra_matrix: d x k projection, rank r, and the (seed, step, id) of A."""
    _fields_ = [("d", ctypes.c_int64), ("k", ctypes.c_int64), ("r", ctypes.c_int64),
                ("seed", ctypes.c_uint64), ("step", ctypes.c_uint64),
                ("matrix_id", ctypes.c_uint64)]

    def __init__(self, d, k, r, seed=0, step=0, matrix_id=0):
        super().__init__(int(d), int(k), int(r), int(seed), int(step), int(matrix_id))


class LaunchOpts(ctypes.Structure):
    """logra_launch_opts: per-call scheduling hints, the fold's wait guard and
    where the backward call runs its fold (0 = default for each field). fold_timeouts may be given as an
    int32 device tensor of one element (or a raw device address); every fold
    workgroup that gives up on its partner adds 1 to it."""
    _fields_ = [("sketch_concurrency", ctypes.c_int32), ("apply_concurrency", ctypes.c_int32),
                ("fold_wait_limit", ctypes.c_int32), ("backward_fold", ctypes.c_int32),
                ("fold_timeouts", ctypes.c_void_p)]

    def __init__(self, sketch_concurrency=0, apply_concurrency=0, fold_wait_limit=0,
                 fold_timeouts=None, backward_fold=0):
        addr = None
        if fold_timeouts is not None:
            if isinstance(fold_timeouts, torch.Tensor):
                if fold_timeouts.dtype != torch.int32 or fold_timeouts.numel() < 1:
                    raise LograError(1, "fold_timeouts: one-element int32 device tensor expected")
                addr = fold_timeouts.data_ptr()
            else:
                addr = int(fold_timeouts)
        super().__init__(int(sketch_concurrency), int(apply_concurrency), int(fold_wait_limit),
                         int(backward_fold), addr)


class KLBudget(ctypes.Structure):
    """logra_kl_budget: KL budget annealed linearly from delta_start to
    delta_end over anneal_steps steps."""
    _fields_ = [("delta_start", ctypes.c_double), ("delta_end", ctypes.c_double),
                ("anneal_steps", ctypes.c_uint64)]

    def __init__(self, delta_start, delta_end, anneal_steps=0):
        super().__init__(float(delta_start), float(delta_end), int(anneal_steps))


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LograError(-1, "load liblogra.so (not built: run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, u64, f32, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_float, ctypes.c_int, ctypes.c_size_t)
    D = ctypes.POINTER(MatrixDesc)
    O = ctypes.POINTER(LaunchOpts)
    lib.logra_abi_version.restype = i32
    lib.logra_abi_version.argtypes = []
    lib.logra_status_string.restype = ctypes.c_char_p
    lib.logra_status_string.argtypes = [i32]
    lib.logra_sign_words.restype = i32
    lib.logra_sign_words.argtypes = [D, P, P]
    lib.logra_sketch_workspace_bytes.restype = sz
    lib.logra_sketch_workspace_bytes.argtypes = [D, i64, i32]
    lib.logra_sketch_accumulate.restype = i32
    lib.logra_sketch_accumulate.argtypes = [D, i64, i32, P, i64, P, i64, P, i32, P, sz, O, P]
    lib.logra_sketch_project.restype = i32
    lib.logra_sketch_project.argtypes = [D, i64, i32, P, i64, P, sz, O, P]
    lib.logra_sketch_fold.restype = i32
    lib.logra_sketch_fold.argtypes = [D, i64, i32, P, i64, P, i32, P, sz, O, P]
    lib.logra_sketch_parts_bytes.restype = sz
    lib.logra_sketch_parts_bytes.argtypes = [D, i64, i32]
    lib.logra_sketch_fold_parts.restype = i32
    lib.logra_sketch_fold_parts.argtypes = [D, i64, i32, P, i64, P, P, sz, i32, P, sz, O, P]
    lib.logra_backward_dx.restype = i32
    lib.logra_backward_dx.argtypes = [D, i64, i32, P, i64, P, i64, P, i64, O, P]
    lib.logra_backward_dx_sketch.restype = i32
    lib.logra_backward_dx_sketch.argtypes = [D, i64, i32, P, i64, P, i64, P, i64, P, i32, P, sz, O, P]
    lib.logra_sqnorm_workspace_bytes.restype = sz
    lib.logra_sqnorm_workspace_bytes.argtypes = [D, i32]
    lib.logra_update_sqnorm.restype = i32
    lib.logra_update_sqnorm.argtypes = [D, i32, P, P, f32, f32, P, P, P, P, sz, P]
    lib.logra_update_sqnorm_prepared.restype = i32
    lib.logra_update_sqnorm_prepared.argtypes = [D, i32, P, P, f32, f32, P, P, P, P, sz, P]
    lib.logra_update_sqnorm_noalloc.restype = i32
    lib.logra_update_sqnorm_noalloc.argtypes = [D, i32, P, P, f32, f32, P, P, P, P]
    lib.logra_sqnorm_prepare.restype = i32
    lib.logra_sqnorm_prepare.argtypes = [D, i32, P, sz, P]
    lib.logra_rowadam_apply.restype = i32
    lib.logra_rowadam_apply.argtypes = [D, i32, P, P, P, i32, i64, f32, f32, f32, O, P]
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.logra_sqnorm_batch_workspace_bytes.restype = sz
    lib.logra_sqnorm_batch_workspace_bytes.argtypes = [i32, D, i32]
    lib.logra_update_sqnorm_batch.restype = i32
    lib.logra_update_sqnorm_batch.argtypes = [i32, D, i32, PP, PP, f32, f32, PP, PP, P, P, sz, P]
    dbl = ctypes.c_double
    lib.logra_kl_budget_at.restype = dbl
    lib.logra_kl_budget_at.argtypes = [ctypes.POINTER(KLBudget), u64]
    lib.logra_kl_step_scale.restype = i32
    lib.logra_kl_step_scale.argtypes = [P, i64, f32, dbl, dbl, P, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    lib.logra_ts_projection_bytes.restype = sz
    lib.logra_ts_projection_bytes.argtypes = [D, i32]
    lib.logra_ts_make_projection.restype = i32
    lib.logra_ts_make_projection.argtypes = [D, i32, P, sz, P]
    lib.logra_ts_sketch_workspace_bytes.restype = sz
    lib.logra_ts_sketch_workspace_bytes.argtypes = [D, i64]
    lib.logra_ts_sketch_accumulate.restype = i32
    lib.logra_ts_sketch_accumulate.argtypes = [D, i64, P, i64, P, i64, P, P, P, P, i32, P, sz, O, P]
    lib.logra_ts_update_workspace_bytes.restype = sz
    lib.logra_ts_update_workspace_bytes.argtypes = [D]
    lib.logra_ts_update.restype = i32
    lib.logra_ts_update.argtypes = [D, P, P, P, P, P, P, P, f32, f32, f32, P, P, sz, P]
    lib.logra_ts_apply.restype = i32
    lib.logra_ts_apply.argtypes = [D, P, sz, P, i32, i64, f32, f32, P]
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise LograError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LOGRA_BF16
    if t.dtype == torch.float32:
        return LOGRA_F32
    raise LograError(2, "dtype %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise LograError(1, "2-D tensor with unit column stride expected")
    return t.stride(0)


def _opts(opts):
    return None if opts is None else ctypes.byref(opts)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def logra_abi_version() -> int:
    return int(load_library().logra_abi_version())


def logra_status_string(status: int) -> str:
    return load_library().logra_status_string(int(status)).decode()


def logra_sign_words(m: MatrixDesc, words: torch.Tensor, stream=None) -> None:
    """words: int64/uint64 device tensor of r * ceil(k/64) elements."""
    _check(load_library().logra_sign_words(ctypes.byref(m), _ptr(words), _stream(stream)),
           "logra_sign_words")


def logra_sketch_workspace_bytes(m: MatrixDesc, T: int, act_dtype: int) -> int:
    return int(load_library().logra_sketch_workspace_bytes(ctypes.byref(m), int(T), int(act_dtype)))


def logra_sketch_accumulate(m: MatrixDesc, X: torch.Tensor, dY: torch.Tensor, S: torch.Tensor,
                            accumulate: bool, ws: Optional[torch.Tensor] = None,
                            stream=None, opts: Optional[LaunchOpts] = None) -> None:
    """S (+)= dY^T (X A^T) for one microbatch; X is T x k, dY is T x d."""
    T = X.shape[0]
    code = _dtype_code(X)
    ws, ws_bytes = _sketch_ws(m, T, code, S.device, ws)
    _check(load_library().logra_sketch_accumulate(
        ctypes.byref(m), T, code, _ptr(X), _ld(X), _ptr(dY), _ld(dY), _ptr(S),
        1 if accumulate else 0, _ptr(ws), ws_bytes, _opts(opts), _stream(stream)),
        "logra_sketch_accumulate")


def _sketch_ws(m, T, code, device, ws):
    if ws is None:
        nbytes = logra_sketch_workspace_bytes(m, T, code)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def logra_sketch_project(m: MatrixDesc, X: torch.Tensor, ws: torch.Tensor, stream=None,
                         opts: Optional[LaunchOpts] = None) -> None:
    """workspace <- X A^T for one microbatch (first half of sketch_accumulate)."""
    ws, nb = _sketch_ws(m, X.shape[0], _dtype_code(X), X.device, ws)
    _check(load_library().logra_sketch_project(
        ctypes.byref(m), X.shape[0], _dtype_code(X), _ptr(X), _ld(X), _ptr(ws), nb,
        _opts(opts), _stream(stream)), "logra_sketch_project")


def logra_sketch_fold(m: MatrixDesc, dY: torch.Tensor, S: torch.Tensor, accumulate: bool,
                      ws: torch.Tensor, stream=None, opts: Optional[LaunchOpts] = None) -> None:
    """S (+)= dY^T (X A^T) with the projection left in ws by logra_sketch_project."""
    ws, nb = _sketch_ws(m, dY.shape[0], _dtype_code(dY), dY.device, ws)
    _check(load_library().logra_sketch_fold(
        ctypes.byref(m), dY.shape[0], _dtype_code(dY), _ptr(dY), _ld(dY), _ptr(S),
        1 if accumulate else 0, _ptr(ws), nb, _opts(opts), _stream(stream)), "logra_sketch_fold")


LOGRA_FOLD_FIRST = 1
LOGRA_FOLD_LAST = 2


def logra_sketch_parts_bytes(m: MatrixDesc, T: int, act_dtype: int) -> int:
    return int(load_library().logra_sketch_parts_bytes(ctypes.byref(m), T, act_dtype))


def logra_sketch_fold_parts(m: MatrixDesc, dY: torch.Tensor, S: torch.Tensor, parts: Optional[torch.Tensor],
                            phase: int, ws: torch.Tensor, stream=None, opts: Optional[LaunchOpts] = None) -> None:
    """The fold with the step's sketch held as S plus the parts between calls;
    phase LOGRA_FOLD_FIRST / LOGRA_FOLD_LAST / both / 0."""
    ws, nb = _sketch_ws(m, dY.shape[0], _dtype_code(dY), dY.device, ws)
    pb = 0 if parts is None else parts.numel() * parts.element_size()
    _check(load_library().logra_sketch_fold_parts(
        ctypes.byref(m), dY.shape[0], _dtype_code(dY), _ptr(dY), _ld(dY), _ptr(S),
        None if parts is None else _ptr(parts), pb, int(phase), _ptr(ws), nb, _opts(opts), _stream(stream)),
        "logra_sketch_fold_parts")


def logra_backward_dx(m: MatrixDesc, dY: torch.Tensor, W: torch.Tensor, dX: torch.Tensor, stream=None,
                      opts: Optional[LaunchOpts] = None) -> None:
    """dX = dY W (bf16): the backward input gradient of Y = X W^T."""
    _check(load_library().logra_backward_dx(
        ctypes.byref(m), dY.shape[0], _dtype_code(dY), _ptr(dY), _ld(dY), _ptr(W), _ld(W), _ptr(dX), _ld(dX),
        _opts(opts), _stream(stream)), "logra_backward_dx")


def logra_backward_dx_sketch(m: MatrixDesc, dY: torch.Tensor, W: torch.Tensor, dX: torch.Tensor,
                             S: torch.Tensor, accumulate: bool, ws: torch.Tensor, stream=None,
                             opts: Optional[LaunchOpts] = None) -> None:
    """dX = dY W and S (+)= dY^T (X A^T) in one launch, the projection read
    from ws (left there by logra_sketch_project)."""
    _check(load_library().logra_backward_dx_sketch(
        ctypes.byref(m), dY.shape[0], _dtype_code(dY), _ptr(dY), _ld(dY), _ptr(W), _ld(W), _ptr(dX), _ld(dX),
        _ptr(S), 1 if accumulate else 0, _ptr(ws), ws.numel() * ws.element_size(), _opts(opts),
        _stream(stream)), "logra_backward_dx_sketch")


def logra_sqnorm_workspace_bytes(m: MatrixDesc, compute_dtype: int) -> int:
    return int(load_library().logra_sqnorm_workspace_bytes(ctypes.byref(m), int(compute_dtype)))


def logra_update_sqnorm(m: MatrixDesc, compute_dtype: int, S: torch.Tensor, v: torch.Tensor,
                        beta2: float, eps: float, v_new: torch.Tensor, sqnorm: torch.Tensor,
                        rowsq: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """Pass 1: v_new <- beta2 v + (1 - beta2) rowsq / k, sqnorm, and rowsq if given."""
    if ws is None:
        nbytes = logra_sqnorm_workspace_bytes(m, compute_dtype)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=S.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load_library().logra_update_sqnorm(
        ctypes.byref(m), int(compute_dtype), _ptr(S), _ptr(v), float(beta2), float(eps),
        _ptr(v_new), _ptr(rowsq), _ptr(sqnorm), _ptr(ws), ws_bytes, _stream(stream)),
        "logra_update_sqnorm")


NOALLOC_SCRATCH_BYTES = 512 * 1024


def logra_update_sqnorm_noalloc(m: MatrixDesc, compute_dtype: int, S: torch.Tensor, v: torch.Tensor,
                                beta2: float, eps: float, v_new: torch.Tensor, sqnorm: torch.Tensor,
                                rowsq: Optional[torch.Tensor] = None, stream=None) -> None:
    """Pass 1 as logra_update_sqnorm, with the library's own device scratch
    instead of a workspace (nothing is allocated); calls on one device must
    not overlap in time."""
    _check(load_library().logra_update_sqnorm_noalloc(
        ctypes.byref(m), int(compute_dtype), _ptr(S), _ptr(v), float(beta2), float(eps),
        _ptr(v_new), _ptr(rowsq), _ptr(sqnorm), _stream(stream)), "logra_update_sqnorm_noalloc")


def logra_sqnorm_prepare(m: MatrixDesc, compute_dtype: int, ws: torch.Tensor, stream=None) -> None:
    """First half of pass 1: the Gram matrix of the step's signs into ws."""
    _check(load_library().logra_sqnorm_prepare(
        ctypes.byref(m), int(compute_dtype), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "logra_sqnorm_prepare")


def logra_update_sqnorm_prepared(m: MatrixDesc, compute_dtype: int, S: torch.Tensor, v: torch.Tensor,
                                 beta2: float, eps: float, v_new: torch.Tensor, sqnorm: torch.Tensor,
                                 ws: torch.Tensor, rowsq: Optional[torch.Tensor] = None,
                                 stream=None) -> None:
    """Second half of pass 1, reading the Gram matrix logra_sqnorm_prepare
    left in ws; together they are logra_update_sqnorm."""
    _check(load_library().logra_update_sqnorm_prepared(
        ctypes.byref(m), int(compute_dtype), _ptr(S), _ptr(v), float(beta2), float(eps),
        _ptr(v_new), _ptr(rowsq), _ptr(sqnorm), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)), "logra_update_sqnorm_prepared")


def logra_rowadam_apply(m: MatrixDesc, compute_dtype: int, S: torch.Tensor, v_new: torch.Tensor,
                        W: torch.Tensor, lr: float, scale: float, eps: float, stream=None,
                        opts: Optional[LaunchOpts] = None) -> None:
    """Pass 2: W -= lr * scale * (S A) / (sqrt(v_new) + eps), row-wise; writes W only."""
    _check(load_library().logra_rowadam_apply(
        ctypes.byref(m), int(compute_dtype), _ptr(S), _ptr(v_new), _ptr(W),
        _dtype_code(W), _ld(W), float(lr), float(scale), float(eps),
        _opts(opts), _stream(stream)), "logra_rowadam_apply")


def logra_kl_budget_at(budget: KLBudget, step: int) -> float:
    """The annealed KL budget of optimizer step `step` (host)."""
    return float(load_library().logra_kl_budget_at(ctypes.byref(budget), int(step)))


def logra_kl_step_scale(sqnorm, lr: float, fisher_scale: float, delta: float):
    """Host step controller. sqnorm: sequence or array of per-matrix sqnorms.
    Returns (scales as a float32 numpy array, kl_pred, kl_after)."""
    import numpy as np
    q = np.ascontiguousarray(np.asarray(sqnorm, dtype=np.float32).reshape(-1))
    out = np.zeros(q.size, dtype=np.float32)
    kl_pred, kl_after = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(load_library().logra_kl_step_scale(
        q.ctypes.data_as(ctypes.c_void_p), q.size, float(lr), float(fisher_scale), float(delta),
        out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(kl_pred), ctypes.byref(kl_after)),
        "logra_kl_step_scale")
    return out, kl_pred.value, kl_after.value


MAX_BATCH = 16


def _matrix_array(ms):
    arr = (MatrixDesc * len(ms))()
    for i, m in enumerate(ms):
        arr[i] = m
    return arr


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])


def logra_sqnorm_batch_workspace_bytes(ms, compute_dtype: int) -> int:
    return int(load_library().logra_sqnorm_batch_workspace_bytes(len(ms), _matrix_array(ms),
                                                                  int(compute_dtype)))


def logra_update_sqnorm_batch(ms, compute_dtype: int, S, v, beta2: float, eps: float, v_new,
                              sqnorm: torch.Tensor, rowsq=None, ws: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """Pass 1 of several matrices of one rank in one call (lists of tensors;
    sqnorm: device tensor of len(ms) floats)."""
    n = len(ms)
    if ws is None:
        nbytes = logra_sqnorm_batch_workspace_bytes(ms, compute_dtype)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=sqnorm.device)
    ws_bytes = ws.numel() * ws.element_size()
    rq = None if rowsq is None else ctypes.cast(_ptr_array(rowsq), ctypes.POINTER(ctypes.c_void_p))
    _check(load_library().logra_update_sqnorm_batch(
        n, _matrix_array(ms), int(compute_dtype),
        ctypes.cast(_ptr_array(S), ctypes.POINTER(ctypes.c_void_p)),
        ctypes.cast(_ptr_array(v), ctypes.POINTER(ctypes.c_void_p)), float(beta2), float(eps),
        ctypes.cast(_ptr_array(v_new), ctypes.POINTER(ctypes.c_void_p)), rq, _ptr(sqnorm), _ptr(ws),
        ws_bytes, _stream(stream)), "logra_update_sqnorm_batch")


# ---- two-sided sketch variant (rank 32, bf16 activations) ----

def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def logra_ts_projection_bytes(m: MatrixDesc, side: int) -> int:
    return int(load_library().logra_ts_projection_bytes(ctypes.byref(m), int(side)))


def logra_ts_make_projection(m: MatrixDesc, side: int, proj: torch.Tensor, stream=None) -> None:
    """Builds side 0 (P, d x 32) or side 1 (Q, k x 32) of matrix m into proj."""
    _check(load_library().logra_ts_make_projection(ctypes.byref(m), int(side), _ptr(proj), _nbytes(proj),
                                                   _stream(stream)), "logra_ts_make_projection")


def logra_ts_projection_fp32(m: MatrixDesc, side: int, proj: torch.Tensor) -> torch.Tensor:
    """View of the n x 32 fp32 projection at the start of a projection buffer."""
    n = m.d if side == 0 else m.k
    return proj[:n * 32 * 4].view(torch.float32).view(n, 32)


def logra_ts_sketch_workspace_bytes(m: MatrixDesc, T: int) -> int:
    return int(load_library().logra_ts_sketch_workspace_bytes(ctypes.byref(m), int(T)))


def logra_ts_sketch_accumulate(m: MatrixDesc, X: torch.Tensor, dY: torch.Tensor, proj_P: torch.Tensor,
                               proj_Q: torch.Tensor, S_L: torch.Tensor, S_R: torch.Tensor, accumulate: bool,
                               ws: Optional[torch.Tensor] = None, stream=None,
                               opts: Optional[LaunchOpts] = None) -> None:
    """S_L^T (+)= X^T (dY P) (k x 32), S_R (+)= dY^T (X Q) (d x 32)."""
    T = X.shape[0]
    if ws is None:
        ws = torch.empty(max(16, logra_ts_sketch_workspace_bytes(m, T)), dtype=torch.uint8, device=X.device)
    _check(load_library().logra_ts_sketch_accumulate(
        ctypes.byref(m), T, _ptr(X), _ld(X), _ptr(dY), _ld(dY), _ptr(proj_P), _ptr(proj_Q), _ptr(S_L), _ptr(S_R),
        1 if accumulate else 0, _ptr(ws), _nbytes(ws), _opts(opts), _stream(stream)),
        "logra_ts_sketch_accumulate")


def logra_ts_update_workspace_bytes(m: MatrixDesc) -> int:
    return int(load_library().logra_ts_update_workspace_bytes(ctypes.byref(m)))


def logra_ts_update(m: MatrixDesc, S_L, S_R, proj_P, m_L, v_L, m_R, v_R, beta1: float, beta2: float, eps: float,
                    sqnorm: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """Moments in place, the coupling and B = U_R C into ws, sqnorm[0] = ||Ghat||^2."""
    _check(load_library().logra_ts_update(
        ctypes.byref(m), _ptr(S_L), _ptr(S_R), _ptr(proj_P), _ptr(m_L), _ptr(v_L), _ptr(m_R), _ptr(v_R),
        float(beta1), float(beta2), float(eps), _ptr(sqnorm), _ptr(ws), _nbytes(ws), _stream(stream)),
        "logra_ts_update")


def logra_ts_apply(m: MatrixDesc, ws: torch.Tensor, W: torch.Tensor, lr: float, scale: float, stream=None) -> None:
    """W -= lr * scale * Ghat from the workspace of the preceding logra_ts_update."""
    _check(load_library().logra_ts_apply(
        ctypes.byref(m), _ptr(ws), _nbytes(ws), _ptr(W), _dtype_code(W), _ld(W), float(lr), float(scale),
        _stream(stream)), "logra_ts_apply")
