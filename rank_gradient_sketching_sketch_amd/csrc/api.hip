// C ABI of liblogra.so: argument validation, per-step key derivation, work
// planning and kernel dispatch. Declarations and the contract of every entry
// point are in include/logra.h. Nothing here allocates memory or keeps state:
// every buffer, workspace included, comes from the caller.
#include <math.h>

#include <atomic>

#include "../../include/logra.h"
#include "launch.hpp"
#include "signs.hpp"

using namespace logra;

namespace {

// key = h(h(h(seed) ^ step) ^ matrix_id), h(x) = first SplitMix64 output of x.
uint64_t stream_key(uint64_t seed, uint64_t step, uint64_t matrix_id) {
    auto h = [](uint64_t x) { return splitmix_finalize(x + kGolden); };
    return h(h(h(seed) ^ step) ^ matrix_id);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bf16_rank_ok(int64_t r) { return r == 32 || r == 64 || r == 128 || r == 256; }

bool matrix_ok(const logra_matrix *m) {
    return m && m->d > 0 && m->k > 0 && m->r > 0 && m->d <= (1ll << 30) && m->k <= (1ll << 30);
}

logra_status from_hip(hipError_t e) { return e == hipSuccess ? LOGRA_OK : LOGRA_ERR_HIP; }

float inv_sqrt_rank(int64_t r) { return 1.0f / sqrtf(static_cast<float>(r)); }

size_t sqnorm_ws_bytes(const logra_matrix *m, int compute_dtype) {
    if (compute_dtype == LOGRA_BF16) {
        const SqnormPlan p = plan_sqnorm_bf16(m->d, m->k, static_cast<int>(m->r));
        return p.partial_bytes + p.gram_bytes;
    }
    return static_cast<size_t>(apply_blocks_f32(m->d)) * sizeof(float);
}

// Buffer views address at most 2^31 bytes.
bool fits_view(int64_t rows, int64_t ld, int64_t elem) { return rows * ld * elem < (1ll << 31); }

// Launch options with their defaults filled in (NULL = all defaults).
struct Opts {
    int sketch_concurrency = 1;
    int apply_concurrency = 1;
    int backward_fold = 0;
    FoldWait wait;
};

bool read_opts(const logra_launch_opts *o, Opts *out) {
    Opts r;
    if (o) {
        if (o->backward_fold < 0 || o->backward_fold > 2) return false;
        r.backward_fold = o->backward_fold;
        if (o->sketch_concurrency < 0 || o->sketch_concurrency > 256) return false;
        if (o->apply_concurrency < 0 || o->apply_concurrency > 256) return false;
        if (o->sketch_concurrency > 0) r.sketch_concurrency = o->sketch_concurrency;
        if (o->apply_concurrency > 0) r.apply_concurrency = o->apply_concurrency;
        if (o->fold_wait_limit != 0) r.wait.spin_limit = o->fold_wait_limit;
        r.wait.timeouts = o->fold_timeouts;
    }
    *out = r;
    return true;
}

}  // namespace

// Scratch of logra_update_sqnorm_noalloc, for callers that cannot allocate:
// every device the library runs on holds its own copy until the process
// ends, and every call on that device shares it. In host code `scratch`
// names a host-side stand-in, never the device memory: the device address
// comes from hipGetSymbolAddress, once per device, and is kept in
// scratch_addr (a cache of a fixed address, written at most once per device
// with the value every caller would write).
constexpr size_t kNoallocScratchBytes = LOGRA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<void *> scratch_addr[kMaxDevices];

// The device address of this device's scratch, or null (with the HIP error
// in *err) if the current device cannot be queried.
static void *device_scratch(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
        if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
        return nullptr;
    }
    scratch_addr[dev].store(p, std::memory_order_release);
    return p;
}

extern "C" {

int logra_abi_version(void) { return LOGRA_ABI_VERSION; }

const char *logra_status_string(int status) {
    switch (status) {
    case LOGRA_OK: return "LOGRA_OK";
    case LOGRA_ERR_INVALID_ARGUMENT: return "LOGRA_ERR_INVALID_ARGUMENT";
    case LOGRA_ERR_UNSUPPORTED: return "LOGRA_ERR_UNSUPPORTED";
    case LOGRA_ERR_WORKSPACE: return "LOGRA_ERR_WORKSPACE";
    case LOGRA_ERR_HIP: return "LOGRA_ERR_HIP";
    default: return "LOGRA_UNKNOWN_STATUS";
    }
}

logra_status logra_sign_words(const logra_matrix *m, uint64_t *words, void *stream) {
    if (!matrix_ok(m) || !words) return LOGRA_ERR_INVALID_ARGUMENT;
    if (m->r > (1ll << 20)) return LOGRA_ERR_UNSUPPORTED;
    const uint64_t key = stream_key(m->seed, m->step, m->matrix_id);
    return from_hip(launch_sign_words(key, static_cast<int>(m->r), static_cast<int>(m->k), words,
                                      static_cast<hipStream_t>(stream)));
}

size_t logra_sketch_workspace_bytes(const logra_matrix *m, int64_t T, int act_dtype) {
    if (!matrix_ok(m) || T < 0) return 0;
    if (T == 0) return 0;
    if (act_dtype == LOGRA_BF16) {
        if (!bf16_rank_ok(m->r)) return 0;
        const Stage1Plan p = plan_stage1_bf16(T, m->k, static_cast<int>(m->r));
        const FoldPlan f = plan_fold_bf16(T, m->d, static_cast<int>(m->r));
        return p.p_bytes + f.xbuf_bytes + f.sync_bytes;
    }
    if (act_dtype == LOGRA_F32) return workspace_sketch_f32(T, m->r);
    return 0;
}

static logra_status check_sketch(const logra_matrix *m, int64_t T, int act_dtype) {
    if (!matrix_ok(m) || T < 0) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype != LOGRA_F32 && act_dtype != LOGRA_BF16) return LOGRA_ERR_UNSUPPORTED;
    if (T > (1ll << 30)) return LOGRA_ERR_UNSUPPORTED;
    if (act_dtype == LOGRA_BF16) {
        if (!bf16_rank_ok(m->r) || m->d % 8 || m->k % 8) return LOGRA_ERR_UNSUPPORTED;
        // the projection (ceil(T/32) blocks of 32 tokens x r, bf16) is read
        // through a 32-bit buffer view
        if (!fits_view(T + 32, m->r, 2)) return LOGRA_ERR_UNSUPPORTED;
    } else if (m->r > 1024) {
        return LOGRA_ERR_UNSUPPORTED;
    }
    return LOGRA_OK;
}

static logra_status check_project(const logra_matrix *m, int64_t T, int act_dtype, const void *X,
                                  int64_t ldx, const void *ws, size_t ws_bytes) {
    if (T == 0) return LOGRA_OK;
    if (!X || ldx < m->k) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype == LOGRA_BF16 && (ldx % 8 || !aligned16(X))) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype == LOGRA_BF16 && !fits_view(T, ldx, 2)) return LOGRA_ERR_UNSUPPORTED;
    const size_t need = logra_sketch_workspace_bytes(m, T, act_dtype);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    return LOGRA_OK;
}

static logra_status check_fold(const logra_matrix *m, int64_t T, int act_dtype, const void *dY,
                               int64_t lddy, const float *S, const void *ws, size_t ws_bytes) {
    if (!S || !aligned16(S)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (T == 0) return LOGRA_OK;
    if (!dY || lddy < m->d) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype == LOGRA_BF16 && (lddy % 8 || !aligned16(dY))) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype == LOGRA_BF16 && (!fits_view(T + 32, lddy, 2) || !fits_view(m->d, m->r, 4 * 16)))
        return LOGRA_ERR_UNSUPPORTED;
    const size_t need = logra_sketch_workspace_bytes(m, T, act_dtype);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    return LOGRA_OK;
}

static hipError_t do_project(const logra_matrix *m, int64_t T, int act_dtype, const void *X,
                             int64_t ldx, void *ws, const Opts &o, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const uint64_t key = stream_key(m->seed, m->step, m->matrix_id);
    const float c = inv_sqrt_rank(m->r);
    const int r = static_cast<int>(m->r);
    if (act_dtype == LOGRA_BF16)
        return launch_project_bf16(r, T, m->d, m->k, key, c, static_cast<const uint16_t *>(X), ldx, ws,
                                   o.sketch_concurrency, st);
    return launch_project_f32(r, T, m->k, key, c, static_cast<const float *>(X), ldx, ws, st);
}

static hipError_t do_fold(const logra_matrix *m, int64_t T, int act_dtype, const void *dY,
                          int64_t lddy, float *S, int accumulate, void *ws, const Opts &o, hipStream_t st) {
    if (T == 0) return accumulate ? hipSuccess : launch_fill_zero(S, m->d * m->r, st);
    const int r = static_cast<int>(m->r);
    if (act_dtype == LOGRA_BF16)
        return launch_fold_bf16(r, T, m->d, m->k, static_cast<const uint16_t *>(dY), lddy, S,
                                accumulate ? 1 : 0, ws, o.wait, st);
    return launch_fold_f32(r, T, m->d, static_cast<const float *>(dY), lddy, S, accumulate ? 1 : 0,
                           ws, st);
}

logra_status logra_sketch_project(const logra_matrix *m, int64_t T, int act_dtype, const void *X,
                                  int64_t ldx, void *ws, size_t ws_bytes, const logra_launch_opts *opts,
                                  void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_sketch(m, T, act_dtype);
    if (e == LOGRA_OK) e = check_project(m, T, act_dtype, X, ldx, ws, ws_bytes);
    if (e != LOGRA_OK) return e;
    return from_hip(do_project(m, T, act_dtype, X, ldx, ws, o, static_cast<hipStream_t>(stream)));
}

logra_status logra_sketch_fold(const logra_matrix *m, int64_t T, int act_dtype, const void *dY,
                               int64_t lddy, float *S, int accumulate, void *ws,
                               size_t ws_bytes, const logra_launch_opts *opts, void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_sketch(m, T, act_dtype);
    if (e == LOGRA_OK) e = check_fold(m, T, act_dtype, dY, lddy, S, ws, ws_bytes);
    if (e != LOGRA_OK) return e;
    return from_hip(do_fold(m, T, act_dtype, dY, lddy, S, accumulate, ws, o,
                            static_cast<hipStream_t>(stream)));
}

size_t logra_sketch_parts_bytes(const logra_matrix *m, int64_t T, int act_dtype) {
    if (check_sketch(m, T, act_dtype) != LOGRA_OK || T == 0 || act_dtype != LOGRA_BF16) return 0;
    return fold_parts_bytes_bf16(T, m->d, static_cast<int>(m->r));
}

logra_status logra_sketch_fold_parts(const logra_matrix *m, int64_t T, int act_dtype, const void *dY,
                                     int64_t lddy, float *S, float *parts, size_t parts_bytes, int phase,
                                     void *ws, size_t ws_bytes, const logra_launch_opts *opts,
                                     void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (phase & ~(LOGRA_FOLD_FIRST | LOGRA_FOLD_LAST)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_sketch(m, T, act_dtype);
    if (e == LOGRA_OK) e = check_fold(m, T, act_dtype, dY, lddy, S, ws, ws_bytes);
    if (e != LOGRA_OK) return e;
    const size_t need = logra_sketch_parts_bytes(m, T, act_dtype);
    if (need > 0) {
        if (!parts || parts_bytes < need) return LOGRA_ERR_WORKSPACE;
        if (!aligned16(parts)) return LOGRA_ERR_INVALID_ARGUMENT;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int accumulate = (phase & LOGRA_FOLD_FIRST) ? 0 : 1;
    if (need == 0) return from_hip(do_fold(m, T, act_dtype, dY, lddy, S, accumulate, ws, o, st));
    return from_hip(launch_fold_parts_ws_bf16(static_cast<int>(m->r), T, m->d, m->k,
                                              static_cast<const uint16_t *>(dY), lddy, S, parts, phase, ws, st));
}

logra_status logra_sketch_accumulate(const logra_matrix *m, int64_t T, int act_dtype,
                                     const void *X, int64_t ldx, const void *dY, int64_t lddy,
                                     float *S, int accumulate, void *ws, size_t ws_bytes,
                                     const logra_launch_opts *opts, void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_sketch(m, T, act_dtype);
    if (e == LOGRA_OK) e = check_fold(m, T, act_dtype, dY, lddy, S, ws, ws_bytes);
    if (e == LOGRA_OK) e = check_project(m, T, act_dtype, X, ldx, ws, ws_bytes);
    if (e != LOGRA_OK) return e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t h = do_project(m, T, act_dtype, X, ldx, ws, o, st);
    if (h != hipSuccess) return LOGRA_ERR_HIP;
    return from_hip(do_fold(m, T, act_dtype, dY, lddy, S, accumulate, ws, o, st));
}

// Arguments of the backward product shared by both entry points.
static logra_status check_dx(const logra_matrix *m, int64_t T, int act_dtype, const void *dY, int64_t lddy,
                             const void *W, int64_t ldw, const void *dX, int64_t lddx) {
    if (!matrix_ok(m) || T < 0) return LOGRA_ERR_INVALID_ARGUMENT;
    if (act_dtype != LOGRA_BF16) return LOGRA_ERR_UNSUPPORTED;
    if (m->d % 8 || m->k % 8 || T > (1ll << 30)) return LOGRA_ERR_UNSUPPORTED;
    if (!W || ldw < m->k || ldw % 8 || !aligned16(W)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!fits_view(m->d, ldw, 2)) return LOGRA_ERR_UNSUPPORTED;
    if (T == 0) return LOGRA_OK;
    if (!dY || lddy < m->d || lddy % 8 || !aligned16(dY)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!dX || lddx < m->k || lddx % 8 || !aligned16(dX)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!fits_view(T, lddy, 2) || !fits_view(T, lddx, 2)) return LOGRA_ERR_UNSUPPORTED;
    return LOGRA_OK;
}

logra_status logra_backward_dx(const logra_matrix *m, int64_t T, int act_dtype, const void *dY, int64_t lddy,
                               const void *W, int64_t ldw, void *dX, int64_t lddx,
                               const logra_launch_opts *opts, void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    const logra_status e = check_dx(m, T, act_dtype, dY, lddy, W, ldw, dX, lddx);
    if (e != LOGRA_OK || T == 0) return e;
    // the r = 256 instance of the launch, the one the fused call runs at the
    // 7B shapes, so the two time the same product code
    return from_hip(launch_dx_bf16(256, T, m->d, m->k, static_cast<const uint16_t *>(dY), lddy,
                                   static_cast<const uint16_t *>(W), ldw, static_cast<uint16_t *>(dX), lddx,
                                   nullptr, 0, nullptr, 0, 0, o.wait, static_cast<hipStream_t>(stream)));
}

logra_status logra_backward_dx_sketch(const logra_matrix *m, int64_t T, int act_dtype, const void *dY,
                                      int64_t lddy, const void *W, int64_t ldw, void *dX, int64_t lddx,
                                      float *S, int accumulate, void *ws, size_t ws_bytes,
                                      const logra_launch_opts *opts, void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_dx(m, T, act_dtype, dY, lddy, W, ldw, dX, lddx);
    if (e == LOGRA_OK) e = check_sketch(m, T, act_dtype);
    if (e == LOGRA_OK) e = check_fold(m, T, act_dtype, dY, lddy, S, ws, ws_bytes);
    if (e != LOGRA_OK) return e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return accumulate ? LOGRA_OK : from_hip(launch_fill_zero(S, m->d * m->r, st));
    const int r = static_cast<int>(m->r);
    const Stage1Plan p = plan_stage1_bf16(T, m->k, r);
    const uint16_t *dy = static_cast<const uint16_t *>(dY);
    const bool fuse = o.backward_fold == 1 || (o.backward_fold == 0 && dx_fuse_pays(T, m->d, m->k, r));
    if (fuse)
        return from_hip(launch_dx_bf16(r, T, m->d, m->k, dy, lddy, static_cast<const uint16_t *>(W), ldw,
                                       static_cast<uint16_t *>(dX), lddx, static_cast<const uint16_t *>(ws),
                                       p.t_blocks, S, accumulate ? 1 : 0, 1, o.wait, st));
    // the fold would outlast the product beside it: the product, then the fold
    if (launch_dx_bf16(r, T, m->d, m->k, dy, lddy, static_cast<const uint16_t *>(W), ldw,
                       static_cast<uint16_t *>(dX), lddx, nullptr, 0, nullptr, 0, 0, o.wait, st) != hipSuccess)
        return LOGRA_ERR_HIP;
    return from_hip(launch_fold_bf16(r, T, m->d, m->k, dy, lddy, S, accumulate ? 1 : 0, ws, o.wait, st));
}

size_t logra_sqnorm_workspace_bytes(const logra_matrix *m, int compute_dtype) {
    if (!matrix_ok(m)) return 0;
    if (compute_dtype != LOGRA_F32 && compute_dtype != LOGRA_BF16) return 0;
    return sqnorm_ws_bytes(m, compute_dtype);
}

static logra_status check_apply_common(const logra_matrix *m, int compute_dtype, const float *S,
                                       float beta2, float eps) {
    if (!matrix_ok(m) || !S) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!(beta2 >= 0.f && beta2 <= 1.f) || !(eps >= 0.f)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (compute_dtype == LOGRA_BF16) {
        if (!bf16_rank_ok(m->r) || m->k % 8) return LOGRA_ERR_UNSUPPORTED;
    } else if (compute_dtype == LOGRA_F32) {
        if (m->r > 1024) return LOGRA_ERR_UNSUPPORTED;
    } else {
        return LOGRA_ERR_UNSUPPORTED;
    }
    if (!aligned16(S)) return LOGRA_ERR_INVALID_ARGUMENT;
    return LOGRA_OK;
}

static ApplyArgs base_args(const logra_matrix *m, const float *S, float beta2, float eps) {
    ApplyArgs a;
    a.R = static_cast<int>(m->r);
    a.D = m->d;
    a.K = m->k;
    a.key = stream_key(m->seed, m->step, m->matrix_id);
    a.c = inv_sqrt_rank(m->r);
    a.S = S;
    a.beta2 = beta2;
    a.eps = eps;
    return a;
}

static logra_status update_sqnorm_parts(const logra_matrix *m, int compute_dtype, const float *S,
                                        const float *v, float beta2, float eps, float *v_new,
                                        float *rowsq, float *sqnorm, void *ws, size_t ws_bytes,
                                        void *stream, int parts);

logra_status logra_update_sqnorm(const logra_matrix *m, int compute_dtype, const float *S,
                                 const float *v, float beta2, float eps, float *v_new,
                                 float *rowsq, float *sqnorm, void *ws, size_t ws_bytes,
                                 void *stream) {
    return update_sqnorm_parts(m, compute_dtype, S, v, beta2, eps, v_new, rowsq, sqnorm, ws, ws_bytes, stream,
                               kSqnormGram | kSqnormRows);
}

logra_status logra_update_sqnorm_prepared(const logra_matrix *m, int compute_dtype, const float *S,
                                          const float *v, float beta2, float eps, float *v_new,
                                          float *rowsq, float *sqnorm, void *ws, size_t ws_bytes,
                                          void *stream) {
    return update_sqnorm_parts(m, compute_dtype, S, v, beta2, eps, v_new, rowsq, sqnorm, ws, ws_bytes, stream,
                               kSqnormRows);
}

logra_status logra_sqnorm_prepare(const logra_matrix *m, int compute_dtype, void *ws, size_t ws_bytes,
                                  void *stream) {
    if (!matrix_ok(m)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (compute_dtype == LOGRA_BF16) {
        if (!bf16_rank_ok(m->r) || m->k % 8) return LOGRA_ERR_UNSUPPORTED;
    } else if (compute_dtype == LOGRA_F32) {
        if (m->r > 1024) return LOGRA_ERR_UNSUPPORTED;
    } else {
        return LOGRA_ERR_UNSUPPORTED;
    }
    const size_t need = sqnorm_ws_bytes(m, compute_dtype);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    if (compute_dtype != LOGRA_BF16) return LOGRA_OK;   // the fp32 pass has nothing to prepare
    ApplyArgs a = base_args(m, nullptr, 0.f, 0.f);
    return from_hip(launch_sqnorm_bf16(a, ws, static_cast<hipStream_t>(stream), kSqnormGram));
}

static logra_status update_sqnorm_parts(const logra_matrix *m, int compute_dtype, const float *S,
                                        const float *v, float beta2, float eps, float *v_new,
                                        float *rowsq, float *sqnorm, void *ws, size_t ws_bytes,
                                        void *stream, int parts) {
    logra_status stt = check_apply_common(m, compute_dtype, S, beta2, eps);
    if (stt != LOGRA_OK) return stt;
    if (!v || !v_new || !sqnorm || v_new == v) return LOGRA_ERR_INVALID_ARGUMENT;
    const size_t need = sqnorm_ws_bytes(m, compute_dtype);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ApplyArgs a = base_args(m, S, beta2, eps);
    a.v_in = v;
    a.v_new_out = v_new;
    a.rowsq_out = rowsq;
    a.sqnorm = sqnorm;
    if (compute_dtype == LOGRA_BF16) return from_hip(launch_sqnorm_bf16(a, ws, st, parts));
    a.partials = static_cast<float *>(ws);
    if (launch_apply_f32(0, a, st) != hipSuccess) return LOGRA_ERR_HIP;
    return from_hip(launch_sqnorm_final(a.partials, apply_blocks_f32(m->d), sqnorm, st));
}

logra_status logra_update_sqnorm_noalloc(const logra_matrix *m, int compute_dtype, const float *S,
                                         const float *v, float beta2, float eps, float *v_new,
                                         float *rowsq, float *sqnorm, void *stream) {
    // the same validation as logra_update_sqnorm, before the scratch is touched
    logra_status stt = check_apply_common(m, compute_dtype, S, beta2, eps);
    if (stt != LOGRA_OK) return stt;
    if (!v || !v_new || !sqnorm || v_new == v) return LOGRA_ERR_INVALID_ARGUMENT;
    const size_t need = sqnorm_ws_bytes(m, compute_dtype);
    if (need > kNoallocScratchBytes) return LOGRA_ERR_WORKSPACE;
    hipError_t e = hipSuccess;
    void *ws = device_scratch(&e);
    if (!ws) return LOGRA_ERR_HIP;
    return update_sqnorm_parts(m, compute_dtype, S, v, beta2, eps, v_new, rowsq, sqnorm, ws, kNoallocScratchBytes,
                               stream, kSqnormGram | kSqnormRows);
}

// Workspace slice of matrix i of a batch: the single-matrix layout, each
// slice 256-byte aligned.
static size_t batch_slice_bytes(const logra_matrix *m, int compute_dtype) {
    return (sqnorm_ws_bytes(m, compute_dtype) + 255) / 256 * 256;
}

size_t logra_sqnorm_batch_workspace_bytes(int n, const logra_matrix *ms, int compute_dtype) {
    if (n < 1 || n > LOGRA_MAX_BATCH || !ms) return 0;
    if (compute_dtype != LOGRA_F32 && compute_dtype != LOGRA_BF16) return 0;
    size_t total = 0;
    for (int i = 0; i < n; ++i) {
        if (!matrix_ok(&ms[i])) return 0;
        total += batch_slice_bytes(&ms[i], compute_dtype);
    }
    return total;
}

logra_status logra_update_sqnorm_batch(int n, const logra_matrix *ms, int compute_dtype,
                                       const float *const *S, const float *const *v, float beta2,
                                       float eps, float *const *v_new, float *const *rowsq,
                                       float *sqnorm, void *ws, size_t ws_bytes, void *stream) {
    if (n < 1 || n > LOGRA_MAX_BATCH || !ms || !S || !v || !v_new || !sqnorm)
        return LOGRA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < n; ++i) {
        const logra_status e = check_apply_common(&ms[i], compute_dtype, S[i], beta2, eps);
        if (e != LOGRA_OK) return e;
        if (ms[i].r != ms[0].r) return LOGRA_ERR_INVALID_ARGUMENT;
        if (!v[i] || !v_new[i] || v_new[i] == v[i]) return LOGRA_ERR_INVALID_ARGUMENT;
    }
    if (!aligned16(sqnorm)) return LOGRA_ERR_INVALID_ARGUMENT;
    const size_t need = logra_sqnorm_batch_workspace_bytes(n, ms, compute_dtype);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    if (compute_dtype == LOGRA_F32) {
        // the fp32 twin: the single-matrix passes one after another
        for (int i = 0; i < n; ++i) {
            ApplyArgs a = base_args(&ms[i], S[i], beta2, eps);
            a.v_in = v[i];
            a.v_new_out = v_new[i];
            a.rowsq_out = rowsq ? rowsq[i] : nullptr;
            a.sqnorm = sqnorm + i;
            a.partials = reinterpret_cast<float *>(base);
            if (launch_apply_f32(0, a, st) != hipSuccess) return LOGRA_ERR_HIP;
            if (launch_sqnorm_final(a.partials, apply_blocks_f32(ms[i].d), a.sqnorm, st) != hipSuccess)
                return LOGRA_ERR_HIP;
            base += batch_slice_bytes(&ms[i], compute_dtype);
        }
        return LOGRA_OK;
    }
    SqnormBatch b;
    b.n = n;
    b.beta2 = beta2;
    b.eps = eps;
    b.sqnorm = sqnorm;
    int wg = 0;
    for (int i = 0; i < n; ++i) {
        const SqnormPlan p = plan_sqnorm_bf16(ms[i].d, ms[i].k, static_cast<int>(ms[i].r));
        SqnormItem &it = b.item[i];
        it.S = S[i];
        it.v = v[i];
        it.v_new = v_new[i];
        it.rowsq = rowsq ? rowsq[i] : nullptr;
        it.slots = reinterpret_cast<uint64_t *>(base);
        it.M = reinterpret_cast<uint16_t *>(base + p.partial_bytes);
        it.key = stream_key(ms[i].seed, ms[i].step, ms[i].matrix_id);
        it.c = inv_sqrt_rank(ms[i].r);
        it.D = static_cast<int>(ms[i].d);
        it.K = static_cast<int>(ms[i].k);
        it.bpw = p.rows_per_block / 16;
        it.wg_begin = wg;
        it.n_wg = p.n_blocks;
        wg += p.n_blocks;
        base += batch_slice_bytes(&ms[i], compute_dtype);
    }
    return from_hip(launch_sqnorm_batch_bf16(static_cast<int>(ms[0].r), b, st));
}

logra_status logra_rowadam_apply(const logra_matrix *m, int compute_dtype, const float *S,
                                 const float *v_new, void *W, int w_dtype, int64_t ldw,
                                 float lr, float scale, float eps, const logra_launch_opts *opts,
                                 void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status stt = check_apply_common(m, compute_dtype, S, 0.f, eps);
    if (stt != LOGRA_OK) return stt;
    if (!v_new || !W) return LOGRA_ERR_INVALID_ARGUMENT;
    if (w_dtype != LOGRA_F32 && w_dtype != LOGRA_BF16) return LOGRA_ERR_UNSUPPORTED;
    if (ldw < m->k) return LOGRA_ERR_INVALID_ARGUMENT;
    if (compute_dtype == LOGRA_BF16 && (ldw % 8 || !aligned16(W))) return LOGRA_ERR_INVALID_ARGUMENT;
    if (compute_dtype == LOGRA_BF16 && !fits_view(m->d, ldw, w_dtype == LOGRA_BF16 ? 2 : 4))
        return LOGRA_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ApplyArgs a = base_args(m, S, 0.f, eps);
    a.v_new_in = v_new;
    a.lr_scale = lr * scale;
    a.W = W;
    a.w_bf16 = w_dtype == LOGRA_BF16 ? 1 : 0;
    a.ldw = ldw;
    return from_hip(compute_dtype == LOGRA_BF16 ? launch_rowadam_bf16(a, o.apply_concurrency, st)
                                                : launch_apply_f32(1, a, st));
}

// ------------------------------------------------------------- two-sided --

// Step value of the projections' streams (side s uses this + s): one the
// sign matrices of a run never take.
constexpr uint64_t kTsProjectionStep = 0xFFFFFFFFFFFFFF00ull;

static logra_status check_ts(const logra_matrix *m) {
    if (!matrix_ok(m)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (m->r != 32 || m->d % 8 || m->k % 8 || m->d < 32 || m->k < 32) return LOGRA_ERR_UNSUPPORTED;
    // the folds' exchange buffers are addressed through 32-bit views
    if (!fits_view(m->d, m->r, 4 * 16) || !fits_view(m->k, m->r, 4 * 16)) return LOGRA_ERR_UNSUPPORTED;
    return LOGRA_OK;
}

size_t logra_ts_projection_bytes(const logra_matrix *m, int side) {
    if (check_ts(m) != LOGRA_OK || (side != 0 && side != 1)) return 0;
    return ts_projection_layout(side ? m->k : m->d).total;
}

logra_status logra_ts_make_projection(const logra_matrix *m, int side, void *proj, size_t proj_bytes,
                                      void *stream) {
    if (side != 0 && side != 1) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_ts(m);
    if (e != LOGRA_OK) return e;
    if (!proj || !aligned16(proj)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (proj_bytes < logra_ts_projection_bytes(m, side)) return LOGRA_ERR_WORKSPACE;
    const uint64_t key = stream_key(m->seed, kTsProjectionStep + static_cast<uint64_t>(side), m->matrix_id);
    return from_hip(launch_ts_projection(key, side ? m->k : m->d, proj, static_cast<hipStream_t>(stream)));
}

size_t logra_ts_sketch_workspace_bytes(const logra_matrix *m, int64_t T) {
    if (check_ts(m) != LOGRA_OK || T <= 0 || T > (1ll << 30)) return 0;
    return ts_sketch_layout(T, m->d, m->k).total;
}

logra_status logra_ts_sketch_accumulate(const logra_matrix *m, int64_t T, const void *X, int64_t ldx,
                                        const void *dY, int64_t lddy, const void *proj_P, const void *proj_Q,
                                        float *S_L, float *S_R, int accumulate, void *ws, size_t ws_bytes,
                                        const logra_launch_opts *opts, void *stream) {
    Opts o;
    if (!read_opts(opts, &o)) return LOGRA_ERR_INVALID_ARGUMENT;
    logra_status e = check_ts(m);
    if (e != LOGRA_OK) return e;
    if (T < 0) return LOGRA_ERR_INVALID_ARGUMENT;
    if (T > (1ll << 30)) return LOGRA_ERR_UNSUPPORTED;
    if (!S_L || !S_R || S_L == S_R || !aligned16(S_L) || !aligned16(S_R)) return LOGRA_ERR_INVALID_ARGUMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (accumulate) return LOGRA_OK;
        if (launch_fill_zero(S_R, m->d * m->r, st) != hipSuccess) return LOGRA_ERR_HIP;
        return from_hip(launch_fill_zero(S_L, m->k * m->r, st));
    }
    if (!X || !dY || !proj_P || !proj_Q || !aligned16(proj_P) || !aligned16(proj_Q)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (ldx < m->k || ldx % 8 || !aligned16(X)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (lddy < m->d || lddy % 8 || !aligned16(dY)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!fits_view(T + 32, ldx, 2) || !fits_view(T + 32, lddy, 2)) return LOGRA_ERR_UNSUPPORTED;
    const size_t need = logra_ts_sketch_workspace_bytes(m, T);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    return from_hip(launch_ts_sketch(T, m->d, m->k, static_cast<const uint16_t *>(X), ldx,
                                     static_cast<const uint16_t *>(dY), lddy, proj_P, proj_Q, S_L, S_R,
                                     accumulate ? 1 : 0, ws, o.wait, st));
}

size_t logra_ts_update_workspace_bytes(const logra_matrix *m) {
    if (check_ts(m) != LOGRA_OK) return 0;
    return ts_update_layout(m->d, m->k).total;
}

logra_status logra_ts_update(const logra_matrix *m, const float *S_L, const float *S_R, const void *proj_P,
                             float *m_L, float *v_L, float *m_R, float *v_R, float beta1, float beta2, float eps,
                             float *sqnorm, void *ws, size_t ws_bytes, void *stream) {
    logra_status e = check_ts(m);
    if (e != LOGRA_OK) return e;
    const void *ptrs[] = {S_L, S_R, proj_P, m_L, v_L, m_R, v_R};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!sqnorm) return LOGRA_ERR_INVALID_ARGUMENT;
    const void *outs[] = {m_L, v_L, m_R, v_R};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (outs[i] == outs[j]) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!(beta1 >= 0.f && beta1 <= 1.f) || !(beta2 >= 0.f && beta2 <= 1.f) || !(eps >= 0.f))
        return LOGRA_ERR_INVALID_ARGUMENT;
    const size_t need = logra_ts_update_workspace_bytes(m);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    return from_hip(launch_ts_update(m->d, m->k, S_L, S_R, proj_P, m_L, v_L, m_R, v_R, beta1, beta2, eps, sqnorm,
                                     ws, static_cast<hipStream_t>(stream)));
}

logra_status logra_ts_apply(const logra_matrix *m, const void *ws, size_t ws_bytes, void *W, int w_dtype,
                            int64_t ldw, float lr, float scale, void *stream) {
    logra_status e = check_ts(m);
    if (e != LOGRA_OK) return e;
    if (!W) return LOGRA_ERR_INVALID_ARGUMENT;
    if (w_dtype != LOGRA_F32 && w_dtype != LOGRA_BF16) return LOGRA_ERR_UNSUPPORTED;
    if (ldw < m->k || ldw % 8 || !aligned16(W)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!isfinite(lr) || !isfinite(scale)) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!fits_view(m->d, ldw, w_dtype == LOGRA_BF16 ? 2 : 4)) return LOGRA_ERR_UNSUPPORTED;
    const size_t need = logra_ts_update_workspace_bytes(m);
    if (!ws || ws_bytes < need || !aligned16(ws)) return LOGRA_ERR_WORKSPACE;
    return from_hip(launch_ts_apply(m->d, m->k, ws, W, w_dtype == LOGRA_BF16 ? 1 : 0, ldw, lr * scale,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
