"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/logra.h declares, and its host-side validation answers without
touching a GPU (every call below returns before any kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logra.h")


@pytest.fixture(scope="module")
def lib():
    from rank_gradient_sketching_sketch_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from rank_gradient_sketching_sketch_amd import build_lib
        build_lib.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(logra_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_entry_points_and_helpers():
    names = declared_functions()
    for n in ("logra_sketch_accumulate", "logra_update_sqnorm", "logra_rowadam_apply",
              "logra_sign_words", "logra_sketch_workspace_bytes", "logra_sqnorm_workspace_bytes",
              "logra_abi_version", "logra_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    from rank_gradient_sketching_sketch_amd import binding as B
    assert B.logra_abi_version() == 5
    assert B.logra_status_string(0) == "LOGRA_OK"
    assert B.logra_status_string(3) == "LOGRA_ERR_WORKSPACE"
    assert B.logra_status_string(99) == "LOGRA_UNKNOWN_STATUS"


def test_no_process_wide_settings(lib):
    # the library keeps no mutable global state: the former process-wide setters
    # are gone, their settings travel with each call in logra_launch_opts
    for name in ("logra_set_fold_wait_limit", "logra_set_sketch_concurrency", "logra_set_apply_concurrency"):
        assert not hasattr(lib, name), name
    src = os.path.join(ROOT, "rank_gradient_sketching_sketch_amd", "csrc")
    for f in sorted(os.listdir(src)):
        for line in open(os.path.join(src, f)):
            # a static declaration that is neither a function nor a constant
            # is mutable state shared by every call; the one exception is the
            # device scratch of the allocation-free pass 1 and the per-device
            # cache of its (fixed) address
            if line.startswith("static ") and "(" not in line.split("=")[0]:
                if f == "api.hip" and re.match(r"static (__device__ __align__\(256\) unsigned char scratch|"
                                               r"std::atomic<void \*> scratch_addr)\[", line):
                    continue
                assert line.startswith(("static constexpr", "static const ")), (f, line)


def test_noalloc_pass1_validation_before_any_device_call(lib):
    # above the scratch limit: WORKSPACE; bad arguments: INVALID_ARGUMENT or
    # UNSUPPORTED; all answered before the device is touched
    from rank_gradient_sketching_sketch_amd import binding as B
    r = ctypes.byref
    V2 = ctypes.c_void_p(0x20000)
    big = B.MatrixDesc(6291456 + 16, 64, 256, 0, 0, 0)
    assert B.logra_sqnorm_workspace_bytes(big, B.LOGRA_BF16) > B.NOALLOC_SCRATCH_BYTES
    ok = B.MatrixDesc(6291456, 64, 256, 0, 0, 0)
    assert B.logra_sqnorm_workspace_bytes(ok, B.LOGRA_BF16) <= B.NOALLOC_SCRATCH_BYTES

    def call(mm, compute=1, beta2=0.9, eps=1e-8, v_new=V2, sqn=FAKE):
        return lib.logra_update_sqnorm_noalloc(r(mm), compute, FAKE, FAKE, ctypes.c_float(beta2),
                                               ctypes.c_float(eps), v_new, None, sqn, None)
    assert call(big) == 3
    assert call(B.MatrixDesc(1048576 + 8, 64, 256, 0, 0, 0), compute=0) == 3
    assert call(ok, beta2=1.5) == 1
    assert call(ok, v_new=FAKE) == 1          # v' must not alias v
    assert call(ok, sqn=None) == 1
    assert call(B.MatrixDesc(64, 64, 48, 0, 0, 0)) == 2
    assert lib.logra_update_sqnorm_noalloc(None, 1, FAKE, FAKE, ctypes.c_float(0.9), ctypes.c_float(1e-8),
                                           V2, None, FAKE, None) == 1


def test_launch_opts_validation(lib):
    # out-of-range hints and fold placements are refused before any launch;
    # NULL and a zeroed struct are the defaults
    from rank_gradient_sketching_sketch_amd import binding as B
    m = _m()
    r = ctypes.byref
    T, ws = 4, 1 << 20

    def acc(o):
        return lib.logra_sketch_accumulate(r(m), T, 1, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, ws, o, None)

    def bad_opts(**kw):
        o = B.LaunchOpts()
        for k, v in kw.items():
            setattr(o, k, v)
        return r(o)

    assert acc(bad_opts(sketch_concurrency=-1)) == 1
    assert acc(bad_opts(sketch_concurrency=257)) == 1
    assert acc(bad_opts(apply_concurrency=300)) == 1
    assert acc(bad_opts(backward_fold=3)) == 1
    assert acc(bad_opts(backward_fold=-1)) == 1
    assert lib.logra_sketch_project(r(m), T, 1, FAKE, 128, FAKE, ws, bad_opts(backward_fold=7), None) == 1
    assert lib.logra_sketch_fold(r(m), T, 1, FAKE, 64, FAKE, 0, FAKE, ws, bad_opts(sketch_concurrency=-5),
                                 None) == 1
    assert lib.logra_rowadam_apply(r(m), 1, FAKE, FAKE, FAKE, 1, 128, ctypes.c_float(1e-3), ctypes.c_float(1.0),
                                   ctypes.c_float(1e-8), bad_opts(apply_concurrency=-1), None) == 1
    # the option checks come first: a bad option with T == 0 (no launch) is still refused
    assert lib.logra_sketch_accumulate(r(m), 0, 1, None, 0, None, 0, FAKE, 1, None, 0,
                                       bad_opts(backward_fold=9), None) == 1
    # valid options with nothing to launch: accepted
    o = B.LaunchOpts(sketch_concurrency=4, apply_concurrency=3, fold_wait_limit=-1, backward_fold=2)
    assert lib.logra_sketch_accumulate(r(m), 0, 1, None, 0, None, 0, FAKE, 1, None, 0, r(o), None) == 0
    assert lib.logra_sketch_accumulate(r(m), 0, 1, None, 0, None, 0, FAKE, 1, None, 0, None, None) == 0


def test_projection_view_overflow_is_unsupported(lib):
    # The projection (ceil(T/32) blocks x 32 tokens x r, bf16) is read through
    # a 32-bit buffer view: with a small d, X and dY fit their views while
    # the projection would not, which must be refused, not wrapped.
    from rank_gradient_sketching_sketch_amd import binding as B
    r = ctypes.byref
    T = (1 << 22)          # 2 * (T + 32) * 256 >= 2^31
    m = B.MatrixDesc(8, 8, 256, 0, 0, 0)
    assert 2 * T * 8 < (1 << 31)                       # X and dY views fit
    assert lib.logra_sketch_accumulate(r(m), T, 1, FAKE, 8, FAKE, 8, FAKE, 0, FAKE, 1 << 40, None, None) == 2
    assert lib.logra_sketch_project(r(m), T, 1, FAKE, 8, FAKE, 1 << 40, None, None) == 2
    assert lib.logra_sketch_fold(r(m), T, 1, FAKE, 8, FAKE, 0, FAKE, 1 << 40, None, None) == 2
    # one 32-token block fewer than the limit needs at r = 256 passes validation
    # up to the workspace check (WORKSPACE: the fake workspace size is too small)
    T_ok = (1 << 22) - 64
    assert lib.logra_sketch_project(r(m), T_ok, 1, FAKE, 8, FAKE, 16, None, None) == 3
    # the same T at r = 128 fits
    m128 = B.MatrixDesc(8, 8, 128, 0, 0, 0)
    assert lib.logra_sketch_project(r(m128), T, 1, FAKE, 8, FAKE, 16, None, None) == 3


def _m(d=64, k=128, r=32):
    from rank_gradient_sketching_sketch_amd import binding as B
    return B.MatrixDesc(d, k, r, 0, 0, 0)


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced by the validation paths


def test_validation_errors_return_before_launch(lib):
    m = _m()
    r = ctypes.byref
    # null descriptor / null S
    assert lib.logra_sketch_accumulate(None, 4, 1, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, 1 << 20, None, None) == 1
    assert lib.logra_sketch_accumulate(r(m), 4, 1, FAKE, 128, FAKE, 64, None, 0, FAKE, 1 << 20, None, None) == 1
    # negative T, ld < cols, misaligned pointer
    assert lib.logra_sketch_accumulate(r(m), -1, 1, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, 1 << 20, None, None) == 1
    assert lib.logra_sketch_accumulate(r(m), 4, 1, FAKE, 100, FAKE, 64, FAKE, 0, FAKE, 1 << 20, None, None) == 1
    assert lib.logra_sketch_accumulate(r(m), 4, 1, ctypes.c_void_p(0x10002), 128, FAKE, 64, FAKE, 0,
                                       FAKE, 1 << 20, None, None) == 1
    # unsupported rank / dtype / shape on the bf16 path
    m48 = _m(r=48)
    assert lib.logra_sketch_accumulate(r(m48), 4, 1, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, 1 << 20, None, None) == 2
    assert lib.logra_sketch_accumulate(r(m), 4, 7, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, 1 << 20, None, None) == 2
    m_odd = _m(d=60)
    assert lib.logra_sketch_accumulate(r(m_odd), 4, 1, FAKE, 128, FAKE, 60, FAKE, 0, FAKE, 1 << 20, None, None) == 2
    # workspace too small / missing
    assert lib.logra_sketch_accumulate(r(m), 4, 1, FAKE, 128, FAKE, 64, FAKE, 0, FAKE, 16, None, None) == 3
    assert lib.logra_sketch_accumulate(r(m), 4, 1, FAKE, 128, FAKE, 64, FAKE, 0, None, 1 << 20, None, None) == 3
    # T == 0 with accumulate: nothing to do, no launch
    assert lib.logra_sketch_accumulate(r(m), 0, 1, None, 0, None, 0, FAKE, 1, None, 0, None, None) == 0
    # apply passes: beta2 out of range, eps < 0, nulls, v' aliasing v, unsupported
    V2 = ctypes.c_void_p(0x20000)
    def sq(beta2, eps, v_new=V2, sqn=FAKE, ws_bytes=1 << 20, mm=m):
        return lib.logra_update_sqnorm(r(mm), 1, FAKE, FAKE, ctypes.c_float(beta2), ctypes.c_float(eps),
                                       v_new, None, sqn, FAKE, ws_bytes, None)
    assert sq(1.5, 1e-8) == 1
    assert sq(0.9, -1.0) == 1
    assert sq(0.9, 1e-8, sqn=None) == 1
    assert sq(0.9, 1e-8, v_new=None) == 1
    assert sq(0.9, 1e-8, v_new=FAKE) == 1          # v' must not alias v
    assert sq(0.9, 1e-8, ws_bytes=0) == 3
    assert sq(0.9, 1e-8, mm=m48) == 2
    assert lib.logra_rowadam_apply(r(m), 1, FAKE, FAKE, FAKE, 1, 100, ctypes.c_float(1e-3),
                                   ctypes.c_float(1.0), ctypes.c_float(1e-8), None, None) == 1
    assert lib.logra_rowadam_apply(r(m), 1, FAKE, None, FAKE, 1, 128, ctypes.c_float(1e-3),
                                   ctypes.c_float(1.0), ctypes.c_float(1e-8), None, None) == 1
    assert lib.logra_rowadam_apply(r(m), 1, FAKE, FAKE, FAKE, 1, 128, ctypes.c_float(1e-3),
                                   ctypes.c_float(1.0), ctypes.c_float(-1.0), None, None) == 1
    assert lib.logra_rowadam_apply(r(m), 1, FAKE, FAKE, FAKE, 5, 128, ctypes.c_float(1e-3),
                                   ctypes.c_float(1.0), ctypes.c_float(1e-8), None, None) == 2
    assert lib.logra_sign_words(None, FAKE, None) == 1


def test_workspace_sizes(lib):
    from rank_gradient_sketching_sketch_amd import binding as B
    m = B.MatrixDesc(18944, 3584, 256)
    ws = B.logra_sketch_workspace_bytes(m, 4096, B.LOGRA_BF16)
    # the projected microbatch X A^T in bf16 (T x r); then, for the two token
    # halves that share each of the 128 tiles of up to 10 x 16 rows, their
    # partial tiles as MFMA fragments (128 x 2 x 160 x r fp32) and their sync
    # words (ticket counter, one counter per workgroup-id group of the 8 XCDs,
    # a flag and an XCD id per tile member, a counter per tile:
    # 1 + 8 + 128 x 5 ints = 2596 bytes, rounded up to 256 bytes)
    assert ws == 4096 * 256 * 2 + 128 * 2 * 160 * 256 * 4 + 2816
    # a small d splits the tokens over more members (8 here), each writing a
    # d x r fp32 partial for the reduction that follows
    small = B.logra_sketch_workspace_bytes(B.MatrixDesc(512, 3584, 256), 4096, B.LOGRA_BF16)
    assert small == 4096 * 256 * 2 + 8 * 512 * 256 * 4
    assert B.logra_sketch_workspace_bytes(m, 0, B.LOGRA_BF16) == 0
    assert B.logra_sketch_workspace_bytes(m, 4096, B.LOGRA_F32) == 4096 * 256 * 4
    assert B.logra_sketch_workspace_bytes(B.MatrixDesc(64, 64, 48), 16, B.LOGRA_BF16) == 0
    # per-workgroup partials of the controller's reduction + the r x r sign Gram matrix (bf16)
    sq = B.logra_sqnorm_workspace_bytes(m, B.LOGRA_BF16)
    assert sq >= 4 * ((18944 + 127) // 128) + 256 * 256 * 2
    assert B.logra_sqnorm_workspace_bytes(m, B.LOGRA_F32) == 4 * ((18944 + 7) // 8)


def test_state_size_is_d_by_r():
    # The sketch state the library keeps per matrix is S (d x r fp32) and v
    # (d fp32): k/r times smaller than a d x k fp32 gradient.
    d, k, r = 18944, 3584, 256
    state = 4 * d * r + 4 * d
    dense = 4 * d * k
    assert abs(dense / (4 * d * r) - k / r) < 1e-12 and state < dense / 13


def test_sqnorm_batch_validation_and_workspace(lib):
    from rank_gradient_sketching_sketch_amd import binding as B
    ms = [B.MatrixDesc(18944, 3584, 256), B.MatrixDesc(512, 3584, 256), B.MatrixDesc(3584, 18944, 256)]
    single = [B.logra_sqnorm_workspace_bytes(m, B.LOGRA_BF16) for m in ms]
    # the single-matrix layouts one after another, each slice 256-byte aligned
    assert B.logra_sqnorm_batch_workspace_bytes(ms, B.LOGRA_BF16) == sum((b + 255) // 256 * 256 for b in single)
    arr = B._matrix_array(ms)
    ptrs = (ctypes.c_void_p * 3)(0x10000, 0x20000, 0x30000)
    vptr = (ctypes.c_void_p * 3)(0x40000, 0x50000, 0x60000)
    vnew = (ctypes.c_void_p * 3)(0x70000, 0x80000, 0x90000)
    PP = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
    call = lambda n, m, vn=vnew, ws=FAKE, wsb=1 << 30: lib.logra_update_sqnorm_batch(
        n, m, 1, PP(ptrs), PP(vptr), ctypes.c_float(0.9), ctypes.c_float(1e-8), PP(vn), None, FAKE, ws, wsb, None)
    assert call(0, arr) == 1                      # n < 1
    assert call(17, arr) == 1                     # n > LOGRA_MAX_BATCH
    assert call(3, arr, vn=vptr) == 1             # v' aliasing v
    assert call(3, arr, wsb=16) == 3              # workspace too small
    assert call(3, arr, ws=None) == 3
    mixed = B._matrix_array([ms[0], B.MatrixDesc(512, 3584, 128), ms[2]])
    assert call(3, mixed) == 1                    # ranks differ
    assert B.logra_sqnorm_batch_workspace_bytes([], B.LOGRA_BF16) == 0


def test_fold_parts_sizes_and_validation(lib):
    # The parts are (n - 1) d x r fp32 where n workgroups share each tile of
    # S: two at the 7B up shape (d = 18944, 4096 tokens), more for small d,
    # one (no parts) for short token counts and on the fp32 path. Bad phases,
    # missing or short parts and misaligned parts are refused before any
    # launch.
    from rank_gradient_sketching_sketch_amd import binding as B
    r = ctypes.byref
    up = B.MatrixDesc(18944, 3584, 256, 0, 0, 0)
    assert B.logra_sketch_parts_bytes(up, 4096, B.LOGRA_BF16) == 18944 * 256 * 4
    assert B.logra_sketch_parts_bytes(up, 4096, B.LOGRA_F32) == 0
    assert B.logra_sketch_parts_bytes(up, 0, B.LOGRA_BF16) == 0
    assert B.logra_sketch_parts_bytes(up, 128, B.LOGRA_BF16) == 0     # 4 steps: one member per tile
    small = B.MatrixDesc(3584, 3584, 256, 0, 0, 0)
    n_small = B.logra_sketch_parts_bytes(small, 4096, B.LOGRA_BF16) // (3584 * 256 * 4)
    assert n_small >= 2
    assert B.logra_sketch_parts_bytes(B.MatrixDesc(18944, 3584, 100, 0, 0, 0), 4096, B.LOGRA_BF16) == 0
    m = B.MatrixDesc(18944, 3584, 256, 0, 0, 0)
    T = 4096
    ws = B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16)
    need = 18944 * 256 * 4

    def call(parts, pb, phase, opts=None):
        return lib.logra_sketch_fold_parts(r(m), T, 1, FAKE, 18944, FAKE, parts, pb, phase, FAKE, ws, opts, None)

    assert call(FAKE, need, 4) == 1
    assert call(FAKE, need, -1) == 1
    assert call(None, 0, 0) == 3
    assert call(FAKE, need - 16, 1) == 3
    assert call(ctypes.c_void_p(0x10008), need, 0) == 1
    o = B.LaunchOpts()
    o.sketch_concurrency = -2
    assert call(FAKE, need, 0, r(o)) == 1
    # the fold's own checks apply too (lddy < d)
    assert lib.logra_sketch_fold_parts(r(m), T, 1, FAKE, 64, FAKE, FAKE, need, 0, FAKE, ws, None, None) == 1
    # T == 0 in a middle microbatch launches nothing and needs no parts
    assert lib.logra_sketch_fold_parts(r(m), 0, 1, None, 0, FAKE, None, 0, 0, None, 0, None, None) == 0


def test_per_file_build_flags_name_sources_that_exist():
    # the fold's register form is set per translation unit; a renamed source
    # would silently lose its flags
    from rank_gradient_sketching_sketch_amd import build_lib
    for name, flags in build_lib.FILE_FLAGS.items():
        assert os.path.exists(os.path.join(build_lib.CSRC, name)), name
        assert flags and all(isinstance(f, str) for f in flags)


def test_pair_mode_fold_instances_live_only_in_their_own_source():
    # the pair-mode fold kernels are built without the fold file's register
    # flag, so no other source may instantiate them
    csrc = os.path.join(ROOT, "rank_gradient_sketching_sketch_amd", "csrc")
    users = [f for f in os.listdir(csrc) if f.endswith(".hip")
             and re.search(r"fold_bf16_kernel<[^>]*kFoldPair>", open(os.path.join(csrc, f)).read())]
    assert users == ["fold_pair_bf16.hip"]
