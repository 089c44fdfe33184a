/*
 * oracle.c -- plain, slow, fp64 CPU reference of LoGRA's sketch-accumulate
 * and RowAdam-apply path.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers. The HIP library never
 * loads this file's library, and the two share no source: the counter hash,
 * the loops and the build line (gcc, not hipcc) here are written separately.
 *
 * Sources (the pages on LoGRA; cited per function below):
 *   [NEWS]  "NVIDIA's LoGRA fits RL post-training of a 27B model onto a
 *           single eight-GPU node" (theclarity.today), sections
 *           "What happened" and "Why it matters".
 *   [DAIR]  "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
 *           Sketches" (academy.dair.ai), paragraphs "Gradient sketches.",
 *           "Step control." and the Abstract.
 *   [AITOP] "NVIDIA LoGRA Paper Cuts RL Training Memory Below LoRA Levels"
 *           (aitop.news), the single item.
 *
 * What is computed, in the pages' order:
 *   A        r x k, A[l][j] = s(l,j) / sqrt(r), s = +-1 from a counter hash
 *            of (seed, step, matrix id); fixed within a step     [DAIR]
 *   P        = X A^T               (T x r) for one microbatch    [NEWS]
 *   S       += dY^T P              (d x r), i.e. S = G A^T with
 *                                  G = dY^T X never formed       [NEWS]
 *   Ghat     = S A                 (d x k), at update time only  [NEWS]
 *   rowsq_i  = sum_j Ghat_ij^2
 *   v'_i     = beta2 v_i + (1 - beta2) rowsq_i / k   (row second moment,
 *                                  no first moment)              [NEWS]
 *   u_i      = 1 / (sqrt(v'_i) + eps)
 *   sqnorm   = sum_ij (Ghat_ij u_i)^2, the quantity a step controller
 *                                  reads before the update       [DAIR]
 *   W'_ij    = W_ij - lr * scale * Ghat_ij * u_i
 *   dX       = dY W               (T x k), the backward input gradient
 *                                  computed from the same dY     [NEWS]
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes): the hash is SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) keyed as
 * described at oracle_stream_key; bit 1 means -1; no bias correction, no
 * weight decay; eps is added to sqrt(v'); the mean over j divides by k;
 * S starts at zero each step.
 *
 * Everything is fp64 with plain loops. OpenMP only splits independent rows
 * (or token rows of P) across threads; each sum runs in index order inside
 * one thread, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of later OpenMP loops (for timing only; n < 1 is
 * ignored). No arithmetic depends on it: every output element is computed
 * by one thread in a fixed order. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- hash --- */

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

/* The SplitMix64 output function (finalizer) applied to one state value. */
uint64_t oracle_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Output number n (n >= 1) of a SplitMix64 generator whose state starts at
 * `state`: the state advances by the golden-ratio increment before each
 * output, so output n mixes state + n * gamma. */
uint64_t oracle_splitmix64_output(uint64_t state, uint64_t n) {
    return oracle_mix64(state + n * SM64_GAMMA);
}

/* Per-(seed, step, matrix) key. Each stage takes the first SplitMix64 output
 * of the previous value: h(x) = output 1 of SplitMix64(x). The step enters
 * after the seed and the matrix id after the step, so A changes every step
 * [DAIR "Gradient sketches."] and differs between matrices. */
uint64_t oracle_stream_key(uint64_t seed, uint64_t step, uint64_t matrix_id) {
    uint64_t h = oracle_splitmix64_output(seed, 1);
    h = oracle_splitmix64_output(h ^ step, 1);
    h = oracle_splitmix64_output(h ^ matrix_id, 1);
    return h;
}

/* Word (l, b) holds the signs of row l, columns 64b .. 64b+63, one bit per
 * column (bit j mod 64). It is output number ((l << 32) | b) + 1 of the
 * SplitMix64 stream that starts at the key. */
uint64_t oracle_sign_word(uint64_t key, int64_t l, int64_t b) {
    uint64_t counter = (((uint64_t)l << 32) | (uint64_t)b) + 1ULL;
    return oracle_splitmix64_output(key, counter);
}

/* words: r x ceil(k/64), row-major. */
void oracle_sign_words(uint64_t seed, uint64_t step, uint64_t matrix_id,
                       int64_t r, int64_t k, uint64_t *words) {
    uint64_t key = oracle_stream_key(seed, step, matrix_id);
    int64_t nb = (k + 63) / 64;
    for (int64_t l = 0; l < r; ++l)
        for (int64_t b = 0; b < nb; ++b)
            words[l * nb + b] = oracle_sign_word(key, l, b);
}

/* The random-sign projection A (r x k, row-major) with entries +-1/sqrt(r)
 * [DAIR "Gradient sketches."; NEWS "Why it matters" gives A as r-by-k].
 * Bit 1 of the hash gives -1, bit 0 gives +1. */
void oracle_sign_matrix(uint64_t seed, uint64_t step, uint64_t matrix_id,
                        int64_t r, int64_t k, double *A) {
    uint64_t key = oracle_stream_key(seed, step, matrix_id);
    double c = 1.0 / sqrt((double)r);
    for (int64_t l = 0; l < r; ++l)
        for (int64_t j = 0; j < k; ++j) {
            uint64_t w = oracle_sign_word(key, l, j / 64);
            int bit = (int)((w >> (j % 64)) & 1ULL);
            A[l * k + j] = bit ? -c : c;
        }
}

/* -------------------------------------------------------------- sketch --- */

/* P = X A^T for one microbatch: P[t][l] = sum_j X[t][j] A[l][j].
 * X is T x k with row stride ldx; A is r x k; P is T x r.
 * First factor of S = G A^T = dY^T (X A^T) [NEWS "Why it matters"]. */
void oracle_project(int64_t T, int64_t k, int64_t r,
                    const double *X, int64_t ldx, const double *A, double *P) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t l = 0; l < r; ++l) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += X[t * ldx + j] * A[l * k + j];
            P[t * r + l] = acc;
        }
}

/* S rows += dY^T P for the listed rows of S (row independence of the sketch
 * lets a test compute any subset exactly). rows == NULL means rows 0..n-1.
 * S_rows is nrows x r. accumulate == 0 overwrites instead of adding, which is
 * how a step's first microbatch starts S at zero.
 * The sketch is summed as microbatches arrive [AITOP; DAIR "Gradient
 * sketches."]. */
void oracle_sketch_rows(int64_t T, int64_t r, const double *dY, int64_t lddy,
                        const double *P, int64_t nrows, const int64_t *rows,
                        double *S_rows, int accumulate) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t i = rows ? rows[q] : q;
        double *s = S_rows + q * r;
        if (!accumulate)
            for (int64_t l = 0; l < r; ++l) s[l] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double g = dY[t * lddy + i];
            for (int64_t l = 0; l < r; ++l)
                s[l] += g * P[t * r + l];
        }
    }
}

/* Ghat rows = S rows A: the full-size estimate of the gradient rows, rebuilt
 * from the two small factors [NEWS "Why it matters"; AITOP]. */
void oracle_reconstruct_rows(int64_t k, int64_t r, int64_t nrows,
                             const double *S_rows, const double *A,
                             double *Ghat) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nrows; ++q)
        for (int64_t j = 0; j < k; ++j) {
            double acc = 0.0;
            for (int64_t l = 0; l < r; ++l)
                acc += S_rows[q * r + l] * A[l * k + j];
            Ghat[q * k + j] = acc;
        }
}

/* ------------------------------------------------------------- RowAdam --- */

/* One RowAdam step on a set of rows [NEWS "What happened", "Why it
 * matters": a running estimate of squared row magnitudes, no first moment].
 *
 * Inputs (nrows rows each): S_rows (x r), A (r x k), v_in, W_in (x k).
 * Outputs: rowsq (sum_j Ghat^2), v_out (= v'), sqterm (sum_j (Ghat u)^2,
 * computed literally, not from rowsq), W_out (fp64, before any rounding).
 * Returns sum(sqterm) over the given rows, summed in row order: the
 * per-matrix reduction a predicted-KL step controller reads [DAIR "Step
 * control."; NEWS "What happened"].
 * Any output pointer may be NULL to skip it (W_in may be NULL if W_out is).
 */
double oracle_rowadam_rows(int64_t k, int64_t r, int64_t nrows,
                           const double *S_rows, const double *A,
                           const double *v_in, double beta2, double eps,
                           double lr, double scale, const double *W_in,
                           double *W_out, double *rowsq, double *v_out,
                           double *sqterm) {
    double *tmp_sq = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(static)
        for (int64_t q = 0; q < nrows; ++q) {
            /* Ghat row q = S row q times A */
            for (int64_t j = 0; j < k; ++j) {
                double acc = 0.0;
                for (int64_t l = 0; l < r; ++l)
                    acc += S_rows[q * r + l] * A[l * k + j];
                g[j] = acc;
            }
            double ss = 0.0;
            for (int64_t j = 0; j < k; ++j) ss += g[j] * g[j];
            double vn = beta2 * v_in[q] + (1.0 - beta2) * ss / (double)k;
            double u = 1.0 / (sqrt(vn) + eps);
            double st = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                double e = g[j] * u;
                st += e * e;
            }
            if (W_out)
                for (int64_t j = 0; j < k; ++j)
                    W_out[q * k + j] = W_in[q * k + j] - lr * scale * g[j] * u;
            if (rowsq) rowsq[q] = ss;
            if (v_out) v_out[q] = vn;
            if (sqterm) sqterm[q] = st;
            tmp_sq[q] = st;
        }
        free(g);
    }
    double total = 0.0;
    for (int64_t q = 0; q < nrows; ++q) total += tmp_sq[q];
    free(tmp_sq);
    return total;
}

/* ------------------------------------------------------- backward dX --- */

/* dX rows = dY rows W: the input gradient of the sketched projection
 * Y = X W^T, dX[t][j] = sum_i dY[t][i] W[i][j], for the listed token rows
 * (rows == NULL: 0..nrows-1). dY is T x d (row stride lddy), W is d x k
 * (row stride ldw), dX_rows is nrows x k. The backward pass computes it
 * from the same dY that the sketch accumulates into S during
 * backpropagation [NEWS "Why it matters"]. */
void oracle_backward_dx_rows(int64_t d, int64_t k, const double *dY, int64_t lddy,
                             const double *W, int64_t ldw, int64_t nrows,
                             const int64_t *rows, double *dX_rows) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t t = rows ? rows[q] : q;
        double *out = dX_rows + q * k;
        for (int64_t j = 0; j < k; ++j) out[j] = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double g = dY[t * lddy + i];
            for (int64_t j = 0; j < k; ++j)
                out[j] += g * W[i * ldw + j];
        }
    }
}
