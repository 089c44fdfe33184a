/*
 * logra.h -- C ABI of liblogra.so: LoGRA low-rank gradient sketching and
 * RowAdam apply on AMD Instinct MI355X (gfx950).
 *
 * The method (pages on LoGRA: "NVIDIA's LoGRA fits RL post-training of a 27B
 * model onto a single eight-GPU node", sections "What happened" and "Why it
 * matters"; "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
 * Sketches", paragraphs "Gradient sketches." and "Step control."):
 *
 *   For a selected linear projection W (d x k, row-major [out, in]) every
 *   microbatch with activations X (T x k) and output gradients dY (T x d)
 *   adds to a d x r sketch
 *         S += dY^T (X A^T),
 *   so the d x k gradient G = dY^T X is never formed. A = Sigma / sqrt(r) is
 *   an r x k random-sign matrix, redrawn each optimizer step and fixed
 *   within it; it is never stored: every kernel regenerates the signs it
 *   needs from a counter hash of (seed, step, matrix_id). At update time the
 *   estimate Ghat = S A is rebuilt tile by tile, twice:
 *     pass 1 (logra_update_sqnorm): rowsq_i = sum_j Ghat_ij^2, the updated
 *        row second moment v'_i = beta2 v_i + (1 - beta2) rowsq_i / k, and
 *        the controller's reduction sqnorm = sum_ij (Ghat_ij / (sqrt(v'_i)+eps))^2;
 *     pass 2 (logra_rowadam_apply): W_ij -= lr*scale*Ghat_ij / (sqrt(v'_i) + eps).
 *   RowAdam keeps one second moment per row and no first moment. v' is a
 *   separate buffer: the caller keeps it as the next step's v (swap the two
 *   buffers) once it applies the update, and keeps v if it skips it. Pass 2
 *   reads only (S, v', the step's key, lr*scale, eps), so the same call
 *   rebuilds the update on any replica of W that receives those.
 *   A host-side step controller reads sqnorm between the two passes and
 *   picks scale. One is provided (logra_kl_step_scale, host code at the end
 *   of this header); a caller may use any other.
 *
 * Sign hash (fixed so that any implementation reproduces A bit for bit):
 *   mix(z)   : SplitMix64 finaliser, z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *              z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31 (mod 2^64)
 *   h(x)     = mix(x + 0x9E3779B97F4A7C15)
 *   key      = h(h(h(seed) ^ step) ^ matrix_id)
 *   word(l,b)= mix(key + (((l << 32) | b) + 1) * 0x9E3779B97F4A7C15)
 *   Sigma[l][j] = -1 if bit (j mod 64) of word(l, j/64) is 1, else +1.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller (except the
 *     host arrays of the step controller at the end). The library
 *     allocates nothing and keeps no mutable global state: everything a
 *     launch depends on is in its arguments (scheduling hints and the
 *     fold's wait limit included, in a caller-owned logra_launch_opts), so
 *     the calls are reentrant and may be made from several host threads at
 *     once, on the same or different streams.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is
 *     enqueued asynchronously on it; results are visible after the caller
 *     synchronises the stream.
 *   - Arguments are validated before anything is enqueued. On any error
 *     nothing is launched and no output is touched.
 *   - Output buffers must not alias each other or the inputs.
 *   - Non-finite inputs are not checked; they propagate into the outputs.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no atomics in any reduction, fixed summation orders).
 *   - Matrices are row-major with a leading dimension (row stride, in
 *     elements) >= the number of columns.
 */
#ifndef LOGRA_H_
#define LOGRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOGRA_ABI_VERSION 5

typedef enum logra_status {
    LOGRA_OK = 0,
    LOGRA_ERR_INVALID_ARGUMENT = 1, /* null/negative/misaligned/out-of-range */
    LOGRA_ERR_UNSUPPORTED = 2,      /* valid, but outside what the kernels do */
    LOGRA_ERR_WORKSPACE = 3,        /* workspace missing or too small        */
    LOGRA_ERR_HIP = 4               /* a HIP launch reported an error        */
} logra_status;

typedef enum logra_dtype {
    LOGRA_F32 = 0,
    LOGRA_BF16 = 1
} logra_dtype;

/* One sketched matrix in one optimizer step. d = rows of W (output
 * features), k = columns (input features), r = sketch rank. (seed, step,
 * matrix_id) select the sign matrix A of this step. */
typedef struct logra_matrix {
    int64_t d;
    int64_t k;
    int64_t r;
    uint64_t seed;
    uint64_t step;
    uint64_t matrix_id;
} logra_matrix;

/*
 * Per-call launch options (host struct, owned by the caller, read during the
 * call only). Pass NULL for the defaults; a zeroed struct means the same.
 * None of these is an operation of the pages: they steer how this
 * implementation shares the chip and guard its in-kernel exchange.
 *   sketch_concurrency  independent sketch calls (of different matrices)
 *                       the caller keeps in flight at once on separate
 *                       streams, this one included; 0 or 1 = this call runs
 *                       alone. With n > 1 the projection sizes its
 *                       workgroups for a 1/n share of the chip (fewer,
 *                       taller ones, 64 tokens each, never fewer than 128 of
 *                       them): faster when other streams fill the rest of
 *                       the chip, slower when the call has it to itself.
 *                       Results stay within the same tolerance of the
 *                       oracle (the projection's summation order differs
 *                       between the two shapes). Range [0, 256].
 *   apply_concurrency   the same for pass 2 (logra_rowadam_apply): with
 *                       n > 1, the bf16 pass 2 of a large matrix (at least
 *                       1024 tiles of 256 rows x 64 columns) deals its work
 *                       over 128 workgroups instead of 256. Range [0, 256].
 *   fold_wait_limit     polls a fold workgroup makes for the workgroup it
 *                       exchanges partial sums with (bf16 path, tall tiles
 *                       split over two token halves); 0 = the default of
 *                       2^20 (about a second). A workgroup that gives up
 *                       writes its rows of S as NaN instead of waiting
 *                       longer, and counts itself in fold_timeouts. A
 *                       negative value makes every such workgroup give up
 *                       without polling, which forces that path from the
 *                       host (for tests of it).
 *   backward_fold       where logra_backward_dx_sketch runs the fold: 0 =
 *                       the library's choice (in the product's launch when
 *                       it is expected to finish within the product, else
 *                       after it), 1 = in the product's launch, 2 = as the
 *                       sketch's fold kernel after the product. Results are
 *                       the same either way to the oracle's tolerance (dX is
 *                       bit-identical). Other values: INVALID_ARGUMENT.
 *   fold_timeouts       DEVICE pointer to one int32, or NULL. Every fold
 *                       workgroup that gives up adds 1 to it (a device-scope
 *                       atomic add), so a caller can tell a time-out from
 *                       non-finite inputs. The caller zeroes it and reads
 *                       it when it likes; one counter may serve many calls.
 */
typedef struct logra_launch_opts {
    int32_t sketch_concurrency;
    int32_t apply_concurrency;
    int32_t fold_wait_limit;
    int32_t backward_fold;
    int32_t *fold_timeouts;
} logra_launch_opts;

/* ABI version of the loaded library (LOGRA_ABI_VERSION). */
int logra_abi_version(void);

/* Static string naming a status code. Never NULL. */
const char *logra_status_string(int status);

/*
 * logra_sign_words -- write the packed sign words of this step's A.
 * Defines: the counter hash above (A is random-sign, redrawn per step and
 * fixed across the step's microbatches: "LoGRA: Scaling LLM Reinforcement
 * Learning...", paragraph "Gradient sketches.").
 * words: device, r x ceil(k/64) uint64, row-major; words[l*nb + b] =
 *        word(l, b). Bits beyond column k-1 in the last word are hash bits
 *        that no kernel uses.
 * Errors: INVALID_ARGUMENT for m == NULL, words == NULL, d/k/r <= 0.
 */
logra_status logra_sign_words(const logra_matrix *m, uint64_t *words, void *stream);

/*
 * logra_sketch_workspace_bytes -- device workspace that
 * logra_sketch_accumulate needs for these sizes (0 when T == 0). Returns 0
 * and sets nothing for invalid arguments (m NULL, sizes <= 0, T < 0, bad
 * dtype). The workspace holds the projected microbatch X A^T, then the
 * partial tiles that the workgroups sharing a tile of S exchange, then (when
 * two share each tile) a few sync words that the projection zeroes and the
 * fold leaves zero. It is scratch, free to reuse once the call's work has
 * run; two calls that run at the same time need two workspaces.
 */
size_t logra_sketch_workspace_bytes(const logra_matrix *m, int64_t T, int act_dtype);

/*
 * logra_sketch_accumulate -- fold one microbatch into the sketch:
 *        S  = dY^T (X A^T)        (accumulate == 0)
 *        S += dY^T (X A^T)        (accumulate != 0)
 * Defines: S = G A^T with G = dY^T X the d x k weight gradient, accumulated
 * during backpropagation as microbatches arrive ("NVIDIA's LoGRA fits RL
 * post-training...", section "Why it matters"; "LoGRA: Scaling LLM
 * Reinforcement Learning...", paragraph "Gradient sketches.").
 * Arguments:
 *   T        tokens in this microbatch (>= 0). T == 0 leaves S unchanged
 *            (accumulate != 0) or sets it to zero (accumulate == 0).
 *   act_dtype LOGRA_BF16: X, dY are bf16; products run on bf16 MFMA with fp32
 *            accumulation, and X A^T is rounded to bf16 (nearest even)
 *            before the second product. LOGRA_F32: fp32 throughout, no
 *            reduced-precision shortcuts.
 *   X        T x k, row stride ldx >= k.
 *   dY       T x d, row stride lddy >= d.
 *   S        d x r fp32, row-major, stride r; in/out.
 *   ws       device workspace of ws_bytes >= logra_sketch_workspace_bytes().
 *   opts     launch options (see logra_launch_opts), or NULL.
 * Requirements of the bf16 path: r in {32, 64, 128, 256}; d, k, ldx, lddy
 *   multiples of 8; X, dY 16-byte aligned; each of X, dY, the projection
 *   (about T x r bf16) and 64 d x r bytes below 2^31 bytes (the kernels
 *   address them with 32-bit offsets). The fp32 path takes any r in
 *   [1, 1024] and any d, k >= 1. S and ws must be 16-byte aligned.
 * Errors: INVALID_ARGUMENT (null pointer when T > 0, sizes <= 0, T < 0,
 *   ld < cols, misalignment, bad opts), UNSUPPORTED (r or shape outside the
 *   above, unknown dtype), WORKSPACE (ws NULL or ws_bytes too small), HIP.
 */
logra_status logra_sketch_accumulate(const logra_matrix *m, int64_t T, int act_dtype,
                                     const void *X, int64_t ldx,
                                     const void *dY, int64_t lddy,
                                     float *S, int accumulate,
                                     void *ws, size_t ws_bytes,
                                     const logra_launch_opts *opts, void *stream);

/*
 * logra_sketch_project / logra_sketch_fold -- the two halves of
 * logra_sketch_accumulate, for callers that schedule them separately (for
 * example to time them, or to overlap the projection of the next microbatch
 * with the fold of this one on another stream, each with its own workspace).
 * Calling project then fold with the same (m, T, act_dtype) and workspace is
 * exactly logra_sketch_accumulate: same kernels, same results.
 *   project: workspace <- X A^T (bf16 path: rounded to bf16, nearest even;
 *            fp32 path: fp32). Same arguments and errors as accumulate.
 *   fold:    S (+)= dY^T (X A^T) reading the projection from the workspace
 *            (and using the rest of it as scratch). The workspace must hold a
 *            projection of this (m, T, act_dtype) made by
 *            logra_sketch_project; fold does not check that it does. Several
 *            folds may follow one projection, one after another.
 * Sources: as logra_sketch_accumulate (S = G A^T factored as dY^T (X A^T)).
 */
logra_status logra_sketch_project(const logra_matrix *m, int64_t T, int act_dtype,
                                  const void *X, int64_t ldx,
                                  void *ws, size_t ws_bytes,
                                  const logra_launch_opts *opts, void *stream);
logra_status logra_sketch_fold(const logra_matrix *m, int64_t T, int act_dtype,
                               const void *dY, int64_t lddy,
                               float *S, int accumulate,
                               void *ws, size_t ws_bytes,
                               const logra_launch_opts *opts, void *stream);

/*
 * logra_sketch_parts_bytes / logra_sketch_fold_parts -- the fold with the
 * step's sketch kept in parts while its microbatches arrive, so that the
 * workgroups sharing a tile of S neither exchange partial tiles nor wait for
 * each other (the sketch is the same S = G A^T summed over the step's
 * microbatches: "NVIDIA's LoGRA fits RL post-training...", section "Why it
 * matters"; "LoGRA: Scaling LLM Reinforcement Learning...", paragraph
 * "Gradient sketches."; how its sum is held during the step is this
 * library's choice).
 * Between the calls of a step the sketch of the microbatches folded so far
 * is S + part_0 + ... + part_{n-2}, where the parts are n - 1 arrays of
 * d x r fp32 in `parts` and n is the number of workgroups that share each
 * tile of S for this (m, T, act_dtype); the call with LOGRA_FOLD_LAST adds
 * the parts into S (in part order), after which S alone holds the sketch.
 * logra_sketch_parts_bytes returns (n - 1) d r 4 bytes: 0 when one
 * workgroup covers each tile (or on the fp32 path), and then fold_parts is
 * logra_sketch_fold with accumulate = !(phase & LOGRA_FOLD_FIRST). It
 * returns 0 for invalid arguments too.
 * Arguments: as logra_sketch_fold, with
 *   parts    device, parts_bytes >= logra_sketch_parts_bytes(m, T,
 *            act_dtype), 16-byte aligned, caller-owned and kept for the
 *            whole step (one per matrix being accumulated). May be NULL
 *            when that size is 0. Its contents between calls are the
 *            library's.
 *   phase    LOGRA_FOLD_FIRST: the step's first microbatch (S and the
 *            parts are overwritten, nothing is read from them);
 *            LOGRA_FOLD_LAST: the step's last microbatch (the parts are
 *            added into S after the fold); both for a one-microbatch step;
 *            0 for every other microbatch. Other bits: INVALID_ARGUMENT.
 * Every call of a step must use the same (m, T, act_dtype), and the step
 * must start with a LOGRA_FOLD_FIRST call. A logra_sketch_fold or
 * logra_backward_dx_sketch call with accumulate != 0 between them adds its
 * microbatch to S alone, which keeps the sum right. Results are
 * deterministic; they differ from logra_sketch_fold's in summation order
 * only (within the same tolerance of the oracle).
 * Errors: those of logra_sketch_fold; WORKSPACE also for parts NULL or
 *   parts_bytes too small when the size above is not 0; INVALID_ARGUMENT
 *   for misaligned parts or a bad phase.
 */
#define LOGRA_FOLD_FIRST 1
#define LOGRA_FOLD_LAST 2
size_t logra_sketch_parts_bytes(const logra_matrix *m, int64_t T, int act_dtype);
logra_status logra_sketch_fold_parts(const logra_matrix *m, int64_t T, int act_dtype,
                                     const void *dY, int64_t lddy, float *S,
                                     float *parts, size_t parts_bytes, int phase,
                                     void *ws, size_t ws_bytes,
                                     const logra_launch_opts *opts, void *stream);

/*
 * logra_backward_dx -- the backward input gradient of the projection,
 *        dX = dY W        (T x k; W is d x k, the layer computes Y = X W^T),
 * bf16 inputs and output, fp32 accumulation, rounded to bf16 (nearest even).
 * Not an operation of the sketch itself: the product the backward pass
 * computes from the same dY that the sketch accumulates "during
 * backpropagation" ("NVIDIA's LoGRA fits RL post-training...", section "Why
 * it matters"), provided here as the yardstick for, and the product half of,
 * logra_backward_dx_sketch.
 * Arguments:
 *   m        d, k of W (r, seed, step and id are not used here).
 *   T        tokens (rows of dY and dX), >= 0; T == 0 launches nothing.
 *   act_dtype LOGRA_BF16 (the only one supported).
 *   dY       T x d, row stride lddy >= d.    W: d x k, row stride ldw >= k.
 *   dX       T x k, row stride lddx >= k, out (written only).
 *   opts     launch options (none is read by the product), or NULL.
 * Requirements: d, k, lddy, ldw, lddx multiples of 8; dY, W, dX 16-byte
 *   aligned; each of dY, W, dX below 2^31 bytes.
 * Errors: INVALID_ARGUMENT (nulls, T < 0, ld < cols, misalignment, bad
 *   opts), UNSUPPORTED (dtype, shapes above), HIP.
 */
logra_status logra_backward_dx(const logra_matrix *m, int64_t T, int act_dtype,
                               const void *dY, int64_t lddy, const void *W, int64_t ldw,
                               void *dX, int64_t lddx, const logra_launch_opts *opts, void *stream);

/*
 * logra_backward_dx_sketch -- logra_backward_dx and logra_sketch_fold in one
 * launch: dX = dY W and S (+)= dY^T (X A^T), the sketch accumulated during
 * backpropagation next to the input gradient computed from the same dY
 * ("NVIDIA's LoGRA fits RL post-training...", section "Why it matters":
 * S = G A^T accumulated during backpropagation). Most workgroups compute dX
 * on the matrix cores; a few run the fold on the compute units and memory
 * bandwidth the product leaves free. Where the fold would outlast the
 * product beside it (small d: few fold tiles, each over all tokens), the
 * call runs the product and then the sketch's fold kernel instead, one after
 * the other on the stream. dX is bit-identical to logra_backward_dx; S
 * matches logra_sketch_fold to the same tolerance of the oracle (in the one
 * launch its tiles cover all tokens, so its summation order differs).
 * Arguments: as logra_backward_dx, plus
 *   m        the full matrix descriptor (r, seed, step, id of this step).
 *   S        d x r fp32, in/out; accumulate as in logra_sketch_fold.
 *   ws       the sketch workspace holding the projection X A^T of this
 *            microbatch made by logra_sketch_project (the same m, T and
 *            act_dtype); only the projection is read.
 *   opts     launch options (fold_wait_limit and fold_timeouts apply when
 *            the fold runs as its own kernel), or NULL.
 * Requirements and errors: those of logra_backward_dx and logra_sketch_fold
 *   together. T == 0 leaves S unchanged (accumulate != 0) or zeroes it.
 */
logra_status logra_backward_dx_sketch(const logra_matrix *m, int64_t T, int act_dtype,
                                      const void *dY, int64_t lddy, const void *W, int64_t ldw,
                                      void *dX, int64_t lddx, float *S, int accumulate,
                                      void *ws, size_t ws_bytes,
                                      const logra_launch_opts *opts, void *stream);

/*
 * logra_sqnorm_workspace_bytes -- device workspace logra_update_sqnorm needs
 * (per-block partial sums of the sqnorm reduction; on the bf16 path also the
 * r x r Gram matrix of the signs; the call zeroes what must start at zero).
 * 0 for invalid m. Calls that run at the same time need separate workspaces.
 */
size_t logra_sqnorm_workspace_bytes(const logra_matrix *m, int compute_dtype);

/*
 * logra_update_sqnorm -- apply pass 1. Rebuilds Ghat = S A tile by tile and
 * reduces, without changing any input:
 *   rowsq[i] = sum_j Ghat_ij^2                       (d floats, optional)
 *   v_new[i] = beta2 * v[i] + (1 - beta2) * rowsq_i / k        (d floats)
 *   sqnorm[0] = sum_i rowsq_i * u_i^2, u_i = 1/(sqrt(v_new_i) + eps)
 * sum_i rowsq_i u_i^2 equals sum_ij (Ghat_ij u_i)^2 because u is constant
 * along a row. sqnorm is the per-matrix quantity a predicted-KL step
 * controller reads before the update ("LoGRA: Scaling LLM Reinforcement
 * Learning...", paragraph "Step control."; the KL from the sketch alone:
 * "NVIDIA's LoGRA fits RL post-training...", section "Why it matters"). The
 * row second moment is RowAdam's ("What happened" on the same page).
 * Arguments:
 *   compute_dtype LOGRA_BF16: S is rounded to bf16 (nearest even) as the
 *            MFMA operand, fp32 accumulation. LOGRA_F32: fp32 arithmetic.
 *   S        d x r fp32 (stride r). v: d fp32 (current second moment), in.
 *   v_new    d fp32, out (must not alias v).
 *   rowsq    d fp32, out, or NULL when not wanted.
 *   sqnorm   1 fp32 on the device, out.
 *   ws       device workspace of ws_bytes >= logra_sqnorm_workspace_bytes().
 * Requirements: bf16 path r in {32, 64, 128, 256} and k multiple of 8; fp32
 *   path r in [1, 1024]. Pointers 16-byte aligned.
 * Errors: INVALID_ARGUMENT (nulls, sizes, beta2 outside [0,1], eps < 0,
 *   misalignment, v_new == v), UNSUPPORTED, WORKSPACE, HIP.
 */
logra_status logra_update_sqnorm(const logra_matrix *m, int compute_dtype,
                                 const float *S, const float *v,
                                 float beta2, float eps,
                                 float *v_new, float *rowsq, float *sqnorm,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * logra_sqnorm_prepare / logra_update_sqnorm_prepared -- logra_update_sqnorm
 * in two calls. Pass 1 first builds the r x r Gram matrix of the step's signs
 * (Sigma Sigma^T, exact integers), which depends only on (seed, step,
 * matrix_id, k, r) and not on S; prepare writes it into the workspace, so a
 * caller can run it early, for example on another stream while the sketch
 * is still accumulating; update_sqnorm_prepared then runs the rest of pass 1
 * reading it. The pair is logra_update_sqnorm: same kernels, bit-identical
 * outputs.
 *   prepare: m, compute_dtype and ws as for logra_update_sqnorm (the same m,
 *            including d, which fixes the workspace layout). The fp32 path
 *            has nothing to prepare and launches nothing.
 *   prepared: the arguments of logra_update_sqnorm; ws must hold the Gram
 *            matrix that prepare wrote for this m, and the caller orders the
 *            two (same stream, or an event) and does not use ws for
 *            anything else in between.
 * Errors: as logra_update_sqnorm (prepare: INVALID_ARGUMENT, UNSUPPORTED,
 *   WORKSPACE, HIP).
 */
logra_status logra_sqnorm_prepare(const logra_matrix *m, int compute_dtype,
                                  void *ws, size_t ws_bytes, void *stream);
logra_status logra_update_sqnorm_prepared(const logra_matrix *m, int compute_dtype,
                                          const float *S, const float *v,
                                          float beta2, float eps,
                                          float *v_new, float *rowsq, float *sqnorm,
                                          void *ws, size_t ws_bytes, void *stream);

/*
 * logra_update_sqnorm_batch -- pass 1 of n matrices in one call (1 <= n <=
 * LOGRA_MAX_BATCH), exactly what n calls of logra_update_sqnorm would give
 * (same arithmetic, bit-identical outputs), with two kernel launches in all
 * on the bf16 path instead of two per matrix. For the many small
 * projections of a layer (attention's k and v fill a fraction of the chip
 * each) the launches, not the bytes, set the time. Sources: as
 * logra_update_sqnorm.
 * Arguments (host arrays of n entries; the pointers in them are device
 * pointers with the meaning they have in logra_update_sqnorm):
 *   ms       the matrices; all with the same r.
 *   S, v, v_new  per matrix; rowsq NULL (none wanted) or an array whose
 *            entries may be NULL.
 *   sqnorm   n fp32 on the device, out (entry i for matrix i).
 *   ws       device workspace of ws_bytes >= logra_sqnorm_batch_workspace_bytes().
 * Errors: as logra_update_sqnorm for any matrix, and INVALID_ARGUMENT for n
 *   outside [1, LOGRA_MAX_BATCH], NULL arrays or differing r. Nothing is
 *   launched on error.
 */
#define LOGRA_MAX_BATCH 16
size_t logra_sqnorm_batch_workspace_bytes(int n, const logra_matrix *ms, int compute_dtype);
logra_status logra_update_sqnorm_batch(int n, const logra_matrix *ms, int compute_dtype,
                                       const float *const *S, const float *const *v,
                                       float beta2, float eps,
                                       float *const *v_new, float *const *rowsq, float *sqnorm,
                                       void *ws, size_t ws_bytes, void *stream);

/*
 * logra_update_sqnorm_noalloc -- logra_update_sqnorm for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same pass 1, the same kernels and
 * bit-identical outputs, with the workspace taken from a scratch array the
 * library holds in device memory instead of from an argument.
 * Arguments, requirements and errors: as logra_update_sqnorm, without ws and
 * ws_bytes. The call allocates nothing and calls no allocating routine.
 * Limit: the workspace logra_update_sqnorm would need for m
 *   (logra_sqnorm_workspace_bytes(m, compute_dtype)) must not exceed
 *   LOGRA_NOALLOC_SCRATCH_BYTES (512 KiB: on the bf16 path d up to 6,291,456
 *   rows at r = 256 and 8,355,840 at r = 32; on the fp32 path d up to
 *   1,048,576 rows at any r); larger m returns LOGRA_ERR_WORKSPACE and
 *   launches nothing.
 * Sharing: each device holds one copy of the scratch until the process ends,
 *   and every call on that device uses it; the call leaves it ready for the
 *   next one (it zeroes what must start at zero itself). Calls that overlap
 *   in time on one device (other streams, other host threads) race on it
 *   and give undefined results: order them (same stream, or events).
 * Errors: as logra_update_sqnorm; WORKSPACE above the limit; HIP if the
 *   current device cannot be queried.
 */
#define LOGRA_NOALLOC_SCRATCH_BYTES (512u * 1024u)
logra_status logra_update_sqnorm_noalloc(const logra_matrix *m, int compute_dtype,
                                         const float *S, const float *v,
                                         float beta2, float eps,
                                         float *v_new, float *rowsq, float *sqnorm,
                                         void *stream);

/*
 * logra_rowadam_apply -- apply pass 2:
 *   W_ij <- W_ij - lr * scale * Ghat_ij / (sqrt(v_new_i) + eps)
 * with Ghat = S A rebuilt tile by tile and v_new the second moment that
 * logra_update_sqnorm produced for the same S (RowAdam, "NVIDIA's LoGRA fits
 * RL post-training...", sections "What happened" and "Why it matters"; the
 * update is rebuilt from the two small factors at the moment it is applied,
 * same page). scale is the step controller's factor. Nothing but W is
 * written. Because the call needs only (S, v_new, the matrix's seed, step and
 * id, lr*scale, eps), it is also how a copy of W elsewhere (a rollout
 * worker's policy) is brought up to date from the sketch instead of from W
 * itself: the low-rank representations serve policy synchronisation too
 * ("LoGRA: Scaling LLM Reinforcement Learning...", abstract). Identical inputs
 * give bit-identical W on every device of this architecture.
 * Arguments:
 *   compute_dtype as in logra_update_sqnorm.
 *   S        d x r fp32. v_new: d fp32, in.
 *   W        d x k, row stride ldw >= k, dtype w_dtype (fp32 math, stored
 *            back at its dtype; bf16 by round-to-nearest-even), in/out.
 *   opts     launch options (apply_concurrency is the one read here), or NULL.
 * Requirements: as logra_update_sqnorm; bf16 W or bf16 compute also need
 *   ldw multiple of 8, W 16-byte aligned and d x ldw elements of W below
 *   2^31 bytes.
 * Errors: INVALID_ARGUMENT (nulls, eps < 0, ld, misalignment, bad opts),
 *   UNSUPPORTED, HIP.
 */
logra_status logra_rowadam_apply(const logra_matrix *m, int compute_dtype,
                                 const float *S, const float *v_new,
                                 void *W, int w_dtype, int64_t ldw,
                                 float lr, float scale, float eps,
                                 const logra_launch_opts *opts, void *stream);

/*
 * Predicted-KL step control (host side; no device work).
 *
 * Before each update the step is scaled so that the predicted change of the
 * policy stays within a KL budget that is annealed over training ("LoGRA:
 * Scaling LLM Reinforcement Learning...", paragraph "Step control."; the KL
 * is predicted from the sketch itself: "NVIDIA's LoGRA fits RL
 * post-training...", section "Why it matters"; the shrink factor is closed
 * form and applied when the prediction exceeds the budget: the walk-through
 * page on LoGRA, section "Predicted-KL Step Control"). The pages do not give
 * the Fisher weighting or the schedule; the readings taken here:
 *   - local quadratic model with an isotropic Fisher, F = phi I:
 *       KL(dW) = 0.5 * phi * sum over matrices of ||dW||_F^2, and with the
 *       RowAdam update dW = -lr * Ghat / (sqrt(v') + eps) that is
 *       KL = 0.5 * phi * lr^2 * sum_m sqnorm_m  (sqnorm from
 *       logra_update_sqnorm), so KL(gamma dW) = gamma^2 KL(dW);
 *   - one shrink factor per step, gamma = min(1, sqrt(delta_t / KL));
 *   - delta_t annealed linearly from delta_start to delta_end over
 *     anneal_steps steps, constant afterwards.
 */
typedef struct logra_kl_budget {
    double delta_start;     /* budget at step 0 (>= 0, finite)                  */
    double delta_end;       /* budget from step anneal_steps on (>= 0, finite)  */
    uint64_t anneal_steps;  /* length of the linear anneal; 0: delta_end always */
} logra_kl_budget;

/*
 * logra_kl_budget_at -- delta_t = delta_start + (delta_end - delta_start) *
 * step / anneal_steps for step < anneal_steps, delta_end from then on (and
 * always when anneal_steps == 0).
 * Returns NaN for b == NULL or a negative or non-finite budget.
 */
double logra_kl_budget_at(const logra_kl_budget *b, uint64_t step);

/*
 * logra_kl_step_scale -- the step controller's decision for one step.
 *   sqnorm   n host floats, the per-matrix sqnorm of logra_update_sqnorm
 *            (copied to the host). Entries that are negative or not finite
 *            are left out of the prediction and get scale 0 (no update).
 *   lr       the step's learning rate (finite).
 *   fisher_scale  phi > 0 (finite), the isotropic Fisher stand-in.
 *   delta    the budget of this step (>= 0, finite; see logra_kl_budget_at).
 *   scales   n host floats, out: gamma for every kept matrix, 0 otherwise.
 *   kl_pred  host, out: 0.5 * phi * lr^2 * (sum of the kept sqnorm, in
 *            index order, in double).
 *   kl_after host, out (may be NULL): gamma^2 * kl_pred.
 * gamma = 1 when kl_pred <= delta, else sqrt(delta / kl_pred).
 * Errors: INVALID_ARGUMENT for n < 0, NULL sqnorm/scales with n > 0, NULL
 *   kl_pred, or lr, fisher_scale, delta outside the ranges above. Nothing is
 *   written on error.
 */
logra_status logra_kl_step_scale(const float *sqnorm, int64_t n, float lr, double fisher_scale,
                                 double delta, float *scales, double *kl_pred, double *kl_after);

/*
 * Two-sided sketch variant (the walk-through page "LoGRA Cuts LLM RL VRAM by
 * 45.7%: Fit 27B on a Single Node", section "Low-Rank Gradient Sketches via
 * Random Projections"). Instead of one d x r sketch with signs redrawn each
 * step, the gradient G = dY^T X (d x k) of a matrix is kept as two sketches
 * made with FIXED, orthonormalized Gaussian projections P (d x r) and
 * Q (k x r):
 *     S_L = P^T G (r x k),   S_R = G Q (d x r),
 * each with a first and a second moment, and the update is rebuilt from them
 * by pseudo-inverse coupling:
 *     U = m / (sqrt(v) + eps) entrywise (for both sketches),
 *     Ghat = U_R (P^T U_R)^+ U_L,   W -= lr * scale * Ghat.
 * For raw sketches of a gradient of rank <= r, Ghat is the gradient itself.
 * Readings where the page is silent (the library's): the moments are
 * m' = beta1 m + (1 - beta1) S and v' = beta2 v + (1 - beta2) S^2 with no
 * bias correction; the pseudo-inverse drops singular values at most
 * 32 * 2^-23 times the largest (the sketches and moments are fp32 state;
 * where the true coupling matrix is singular an untruncated inverse would be
 * set by their rounding); the Gaussian entries and the projections are fixed
 * as follows.
 *   Gaussian entry (i, j) of side s (0: P, n = d; 1: Q, n = k): with
 *   key = h(h(h(seed) ^ (0xFFFFFFFFFFFFFF00 + s)) ^ matrix_id) (the sign
 *   hash's key with that step value) and out(c) = mix(key + c *
 *   0x9E3779B97F4A7C15), c = 2 (32 i + j) + 1: u1 = ((out(c) >> 11) + 1)
 *   2^-53, u2 = (out(c + 1) >> 11) 2^-53, z = sqrt(-2 ln u1) cos(2 pi u2).
 *   The projection is the Q factor of that n x 32 matrix whose R factor has
 *   a positive diagonal (computed in fp64 and stored in fp32).
 * Only r = 32 (m->r == 32; the page names 16 or 32) and bf16 activations
 * are built; d and k must be multiples of 8, at least 32 and below 2^20
 * (the fold's exchange buffer is addressed through 32-bit views). S_L is stored
 * TRANSPOSED, as a k x 32 fp32 row-major array (S_L^T); S_R is d x 32 fp32.
 * The moments have the shapes of their sketches (m_L, v_L: k x 32; m_R,
 * v_R: d x 32, fp32). m->step is not used: the projections are fixed.
 *
 * logra_ts_projection_bytes -- bytes of the buffer holding one side's
 *   projection (n = d for side 0, n = k for side 1): the n x 32 fp32 matrix
 *   first, then its bf16 copy in the layout the sketch kernels read, then
 *   scratch of its construction. 0 for invalid arguments.
 * logra_ts_make_projection -- builds side `side` (0 or 1) of matrix m into
 *   proj (device, 16-byte aligned, >= logra_ts_projection_bytes bytes).
 *   Done once per matrix; the buffer is read by the calls below and must
 *   not change between them. Errors: INVALID_ARGUMENT (side, null or not
 *   16-byte aligned proj), UNSUPPORTED (r != 32, d or k outside the range
 *   above), WORKSPACE (proj_bytes too small).
 */
size_t logra_ts_projection_bytes(const logra_matrix *m, int side);
logra_status logra_ts_make_projection(const logra_matrix *m, int side, void *proj, size_t proj_bytes,
                                      void *stream);

/*
 * logra_ts_sketch_accumulate -- one microbatch of T tokens:
 *     S_L^T (+)= X^T (dY P)   (k x 32),   S_R (+)= dY^T (X Q)   (d x 32),
 *   "+=" when accumulate != 0, "=" otherwise. X: T x k bf16 (row stride
 *   ldx), dY: T x d bf16 (row stride lddy), both 16-byte aligned with
 *   strides that are multiples of 8. proj_P / proj_Q: the buffers of sides 0
 *   and 1 made by logra_ts_make_projection for this matrix. X Q and dY P are
 *   formed on the matrix cores with fp32 accumulation and rounded to bf16
 *   (the sketch's fold then takes them as operands, as the one-sided path
 *   does with its projection); S is accumulated in fp32.
 *   ws: device, 16-byte aligned, >= logra_ts_sketch_workspace_bytes(m, T).
 *   T = 0 leaves S untouched with accumulate != 0 and zeroes it otherwise.
 *   opts: only fold_wait_limit and fold_timeouts are read (the folds that
 *   split tall tiles over two token halves wait as in the one-sided fold).
 *   Errors: INVALID_ARGUMENT (pointers, strides, alignment), UNSUPPORTED
 *   (r != 32, shapes; views of X, dY past 2^31 bytes), WORKSPACE.
 */
size_t logra_ts_sketch_workspace_bytes(const logra_matrix *m, int64_t T);
logra_status logra_ts_sketch_accumulate(const logra_matrix *m, int64_t T, const void *X, int64_t ldx,
                                        const void *dY, int64_t lddy, const void *proj_P, const void *proj_Q,
                                        float *S_L, float *S_R, int accumulate, void *ws, size_t ws_bytes,
                                        const logra_launch_opts *opts, void *stream);

/*
 * logra_ts_update -- the step-time part before the controller: updates the
 *   four moments in place from S_L^T and S_R, forms U_L, U_R, the coupling
 *   C = (P^T U_R)^+ (fp64 one-sided Jacobi SVD of the 32 x 32 matrix, whose
 *   Gram sums are taken in fp64) and B = U_R C into ws, and writes
 *   sqnorm[0] = ||Ghat||_F^2 (device float; from the fp64 Gram matrices, for
 *   the step controller). beta1, beta2 in [0, 1], eps >= 0.
 *   ws: >= logra_ts_update_workspace_bytes(m) bytes, 16-byte aligned; it
 *   holds what logra_ts_apply reads, so the apply call of this matrix must
 *   come before ws is used again.
 *   Errors: INVALID_ARGUMENT (pointers, aliasing moments, betas, eps),
 *   UNSUPPORTED (r != 32, shapes), WORKSPACE.
 * logra_ts_apply -- W -= lr * scale * Ghat with Ghat = B U_L from the
 *   workspace of the preceding logra_ts_update of this matrix. The products
 *   take each fp32 operand as a bf16 head plus a bf16 tail (three matrix-core
 *   products), close to an fp32 product; W is bf16 (rounded to nearest once)
 *   or fp32, row stride ldw (multiple of 8, 16-byte aligned).
 *   Errors: INVALID_ARGUMENT (pointers, ldw, non-finite lr or scale),
 *   UNSUPPORTED (w_dtype, r != 32, shapes), WORKSPACE.
 */
size_t logra_ts_update_workspace_bytes(const logra_matrix *m);
logra_status logra_ts_update(const logra_matrix *m, const float *S_L, const float *S_R, const void *proj_P,
                             float *m_L, float *v_L, float *m_R, float *v_R, float beta1, float beta2, float eps,
                             float *sqnorm, void *ws, size_t ws_bytes, void *stream);
logra_status logra_ts_apply(const logra_matrix *m, const void *ws, size_t ws_bytes, void *W, int w_dtype,
                            int64_t ldw, float lr, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_H_ */
