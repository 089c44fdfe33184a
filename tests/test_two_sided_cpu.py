"""CPU checks of the two-sided sketch entry points (logra_ts_*): buffer sizes
and the host-side validation, every call returning before any kernel launch."""
import ctypes

import pytest

from rank_gradient_sketching_sketch_amd import binding as B

FAKE = ctypes.c_void_p(0x10000)       # a 16-byte aligned stand-in, never dereferenced
FAKE2 = ctypes.c_void_p(0x20000)
FAKE3 = ctypes.c_void_p(0x30000)
FAKE4 = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10008)        # 8-byte aligned only
r = ctypes.byref
f = ctypes.c_float


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        from rank_gradient_sketching_sketch_amd import build_lib
        build_lib.build()
    return B.load_library()


def _a256(b):
    return (b + 255) // 256 * 256


def test_projection_buffer_size(lib):
    # fp32 n x 32, its bf16 operand copy over whole 32-row blocks, then the
    # fp64 construction scratch: the n x 32 matrix, one 32 x 32 Gram partial
    # per 64-row block, the summed Gram matrix and R^-1
    m = B.MatrixDesc(18944, 3584, 32, seed=1, matrix_id=2)
    for side, n in ((0, 18944), (1, 3584)):
        nb = (n + 63) // 64
        want = (_a256(n * 32 * 4) + _a256((n + 31) // 32 * 32 * 32 * 2) + _a256(n * 32 * 8)
                + _a256(nb * 1024 * 8) + 2 * 8192)
        assert B.logra_ts_projection_bytes(m, side) == want
    assert B.logra_ts_projection_bytes(m, 2) == 0
    assert B.logra_ts_projection_bytes(B.MatrixDesc(18944, 3584, 64), 0) == 0     # rank 32 only
    assert B.logra_ts_projection_bytes(B.MatrixDesc(24, 3584, 32), 0) == 0        # d < 32
    assert B.logra_ts_projection_bytes(B.MatrixDesc(100, 3584, 32), 0) == 0       # d % 8


def test_sketch_workspace_size(lib):
    # Xq and Yp (bf16, T rounded up to 32 tokens, x 32 columns), the fp32
    # partials of the projection kernel (one per 4096-column chunk of X and of
    # dY), then the two folds' own scratch: none for the fold over d = 18944
    # rows (at r = 32 and 4096 tokens its tiles run over all tokens, one
    # workgroup each), one d x 32 fp32 partial per member for the fold over
    # k = 3584 (small d: several members per tile)
    m = B.MatrixDesc(18944, 3584, 32)
    T = 4096
    chunks = (3584 + 4095) // 4096 + (18944 + 4095) // 4096
    base = 2 * T * 32 * 2 + chunks * T * 32 * 4
    ws = B.logra_ts_sketch_workspace_bytes(m, T)
    members = (ws - base) // (3584 * 32 * 4)
    assert ws == base + members * 3584 * 32 * 4 and 2 <= members <= 16
    assert B.logra_ts_sketch_workspace_bytes(m, 0) == 0
    assert B.logra_ts_sketch_workspace_bytes(B.MatrixDesc(18944, 3584, 256), T) == 0
    # ragged T rounds up to whole 32-token blocks
    assert B.logra_ts_sketch_workspace_bytes(m, 4095) == ws


def test_update_workspace_size(lib):
    d, k = 18944, 3584
    m = B.MatrixDesc(d, k, 32)
    nb = (d + 63) // 64 + (k + 63) // 64
    want = (_a256(d * 32 * 4) + _a256(k * 32 * 4) + _a256(d * 32 * 4) + _a256(1024 * 4) + _a256(3 * 1024 * 8)
            + _a256(nb * 2 * 1024 * 8))
    assert B.logra_ts_update_workspace_bytes(m) == want
    assert B.logra_ts_update_workspace_bytes(B.MatrixDesc(d, k, 16)) == 0


def test_make_projection_validation(lib):
    m = B.MatrixDesc(4096, 4096, 32)
    nb = B.logra_ts_projection_bytes(m, 0)
    assert lib.logra_ts_make_projection(None, 0, FAKE, nb, None) == 1
    assert lib.logra_ts_make_projection(r(m), 2, FAKE, nb, None) == 1
    assert lib.logra_ts_make_projection(r(m), 0, None, nb, None) == 1
    assert lib.logra_ts_make_projection(r(m), 0, MIS, nb, None) == 1
    assert lib.logra_ts_make_projection(r(m), 0, FAKE, nb - 1, None) == 3
    assert lib.logra_ts_make_projection(r(B.MatrixDesc(4096, 4096, 16)), 0, FAKE, nb, None) == 2
    assert lib.logra_ts_make_projection(r(B.MatrixDesc(1 << 20, 4096, 32)), 0, FAKE, 1 << 40, None) == 2


def test_sketch_validation(lib):
    m = B.MatrixDesc(512, 256, 32)
    T = 100
    ws = B.logra_ts_sketch_workspace_bytes(m, T)

    def call(mm=m, T=T, X=FAKE, ldx=256, dY=FAKE2, lddy=512, P=FAKE3, Q=FAKE4, SL=FAKE, SR=FAKE2, acc=0,
             w=FAKE3, wb=ws, opts=None):
        return lib.logra_ts_sketch_accumulate(r(mm), T, X, ldx, dY, lddy, P, Q, SL, SR, acc, w, wb, opts, None)

    assert call(T=-1) == 1
    assert call(SL=None) == 1
    assert call(SL=FAKE2, SR=FAKE2) == 1                 # S_L aliasing S_R
    assert call(SR=MIS) == 1
    assert call(X=None) == 1
    assert call(P=None) == 1
    assert call(Q=MIS) == 1
    assert call(ldx=255) == 1
    assert call(ldx=260) == 1                           # stride not a multiple of 8
    assert call(lddy=504) == 1
    assert call(X=MIS) == 1
    assert call(mm=B.MatrixDesc(512, 256, 64)) == 2
    assert call(mm=B.MatrixDesc(512, 260, 32), ldx=264) == 2
    assert call(wb=ws - 16) == 3
    assert call(w=None) == 3
    assert call(T=(1 << 30) + 1) == 2
    assert call(ldx=1 << 24, T=200) == 2                 # X view past 2^31 bytes
    o = B.LaunchOpts()
    o.backward_fold = 7
    assert call(opts=r(o)) == 1
    # T == 0 with accumulate: nothing to do, no launch, no buffers needed
    assert call(T=0, X=None, dY=None, P=None, Q=None, w=None, wb=0, acc=1) == 0


def test_update_and_apply_validation(lib):
    m = B.MatrixDesc(512, 256, 32)
    wsb = B.logra_ts_update_workspace_bytes(m)
    ptr = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]

    def upd(mm=m, SL=ptr[0], SR=ptr[1], P=ptr[2], mL=ptr[3], vL=ptr[4], mR=ptr[5], vR=ptr[6], b1=0.9, b2=0.99,
            eps=1e-8, sq=ptr[7], w=FAKE, wb=wsb):
        return lib.logra_ts_update(r(mm), SL, SR, P, mL, vL, mR, vR, f(b1), f(b2), f(eps), sq, w, wb, None)

    assert upd(SL=None) == 1
    assert upd(P=MIS) == 1
    assert upd(sq=None) == 1
    assert upd(vR=ptr[3]) == 1                           # moments aliasing
    assert upd(b1=1.5) == 1
    assert upd(b2=-0.1) == 1
    assert upd(eps=-1.0) == 1
    assert upd(b1=float("nan")) == 1
    assert upd(mm=B.MatrixDesc(512, 256, 16)) == 2
    assert upd(wb=wsb - 1) == 3
    assert upd(w=None) == 3

    def app(mm=m, w=FAKE, wb=wsb, W=FAKE2, dt=1, ldw=256, lr=1e-3, sc=1.0):
        return lib.logra_ts_apply(r(mm), w, wb, W, dt, ldw, f(lr), f(sc), None)

    assert app(W=None) == 1
    assert app(dt=5) == 2
    assert app(ldw=252) == 1
    assert app(ldw=260) == 1
    assert app(W=MIS) == 1
    assert app(lr=float("inf")) == 1
    assert app(sc=float("nan")) == 1
    assert app(wb=wsb - 1) == 3
    assert app(mm=B.MatrixDesc(512, 256, 64)) == 2
    assert app(ldw=1 << 22, dt=0) == 2                   # W view past 2^31 bytes
