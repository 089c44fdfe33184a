// The two-sided sketch variant, bf16 activations, rank 32.
//
// The walk-through page "LoGRA Cuts LLM RL VRAM by 45.7%: Fit 27B on a Single
// Node" (section "Low-Rank Gradient Sketches via Random Projections")
// describes LoGRA with two fixed, orthonormalized random Gaussian projections
// P (d x r) and Q (k x r), rank 16 or 32, two sketches of the gradient
// G = dY^T X (d x k),
//     S_L = P^T G (r x k, kept here transposed as k x r)   S_R = G Q (d x r),
// first and second moments of both, and an update rebuilt by pseudo-inverse
// coupling of the two sketches, G_hat = U_R (P^T U_R)^+ U_L with
// U = m / (sqrt(v) + eps) entrywise. The other pages describe one-sided
// random-sign sketches with no first moment (the main path of this library);
// this file builds the variant as that page states it, at r = 32.
//
// Kernels:
//   * projections (once per matrix; they are fixed): Gaussian entries from
//     the counter hash (Box-Muller on two SplitMix64 outputs, fp64) and the Q
//     factor with a positive-diagonal R by two passes of Cholesky QR (for an
//     n x 32 Gaussian matrix with n >> 32 the Gram matrix is well
//     conditioned, and the second pass restores orthogonality to working
//     precision), all in fp64: Gram partials per 64-row block, a tree sum,
//     one workgroup for the Cholesky factor and R^-1, products with R^-1 per
//     block. Kept in fp32 and in the bf16 operand layout of the projection
//     kernel.
//   * sketch (per microbatch): Xq = X Q and Yp = dY P on the matrix cores
//     (bf16 operands, fp32 accumulation) as fp32 partials over column chunks
//     of X and dY, added in chunk order and rounded to bf16 in the fold's
//     operand layout; then the sketch's own fold kernel twice:
//     S_R (+)= dY^T Xq and S_L^T (+)= X^T Yp.
//   * update (per step): moments of both sketches and the normalized sketches
//     with per-block fp64 partials of U_R^T U_R, P^T U_R and U_L U_L^T; a tree
//     sum; one workgroup for the pseudo-inverse C of the 32 x 32 coupling
//     matrix M by cyclic one-sided Jacobi on its columns (fp64; singular
//     values at most 32 times the fp32 machine
//     epsilon 2^-23 times the largest count as zero: the sketches and
//     moments are fp32, and where the true coupling matrix is singular an
//     untruncated inverse would be set by their rounding) and the squared
//     norm of G_hat from the three Gram matrices
//     (||U_R C U_L||^2 = sum (C^T (U_R^T U_R) C) o (U_L U_L^T));
//     then B = U_R C (d x 32, fp32).
//   * apply: W -= step B U_L over 128 x 128 tiles on the matrix cores, each
//     fp32 operand split into a bf16 head and a bf16 tail (three products:
//     head x head, head x tail, tail x head, close to fp32 accuracy), staged in
//     LDS so W moves in whole 16-byte pieces of rows.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

constexpr int kTsR = 32;              // the rank this path is built for
constexpr int kTsRows = 64;           // rows per workgroup of the row kernels
constexpr int kTsGram = kTsR * kTsR;
constexpr int kTsChunkSteps = 128;    // 32-column steps of X or dY per projection workgroup (8 waves x 16)

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// ------------------------------------------------------- block partial sum --

// dst[e] = sum over blocks w = begin .. begin + count - 1 (in order within
// each of four interleaved groups, then the groups in order) of
// src[w * stride + e], e < 1024. grid (16, jobs), 256 threads.
struct TsSumJob {
    const double *src;
    int64_t stride;
    int begin, count;
    double *dst;
};
struct TsSumArgs {
    TsSumJob job[3];
};

__global__ __launch_bounds__(256) void ts_sum_kernel(TsSumArgs a) {
    __shared__ double red[4][64];
    const TsSumJob &j = a.job[blockIdx.y];
    const int tid = threadIdx.x, grp = tid >> 6;
    const int e = 64 * blockIdx.x + (tid & 63);
    double s = 0.0;
#pragma unroll 8
    for (int w = grp; w < j.count; w += 4) s += j.src[static_cast<int64_t>(j.begin + w) * j.stride + e];
    red[grp][tid & 63] = s;
    __syncthreads();
    if (tid < 64) j.dst[e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

static hipError_t launch_sum(const TsSumArgs &a, int jobs, hipStream_t st) {
    hipLaunchKernelGGL(ts_sum_kernel, dim3(kTsGram / 64, jobs), dim3(256), 0, st, a);
    return hipGetLastError();
}

// Gram partial of a kTsRows x 32 tile held in LDS: out[a][b] = sum over the
// tile's rows of x[i][a] y[i][b] (fp64, row order); 256 threads.
template <typename TX, typename TY>
__device__ __forceinline__ void ts_tile_gram(const TX (*x)[kTsR + 1], const TY (*y)[kTsR + 1], int rows,
                                             double *__restrict__ out) {
    const int tid = threadIdx.x;
    const int a = tid >> 3, b0 = 4 * (tid & 7);
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int i = 0; i < rows; ++i) {
        const double xv = x[i][a];
        s0 += xv * static_cast<double>(y[i][b0]);
        s1 += xv * static_cast<double>(y[i][b0 + 1]);
        s2 += xv * static_cast<double>(y[i][b0 + 2]);
        s3 += xv * static_cast<double>(y[i][b0 + 3]);
    }
    out[a * kTsR + b0] = s0;
    out[a * kTsR + b0 + 1] = s1;
    out[a * kTsR + b0 + 2] = s2;
    out[a * kTsR + b0 + 3] = s3;
}

// ------------------------------------------------------------ projections --

// Standard normal entry (i, j) of an n x 32 matrix: outputs 2 (32 i + j) + 1
// and + 2 of the side's stream, u1 in (0, 1], u2 in [0, 1), cosine branch.
__device__ __forceinline__ double ts_gaussian(uint64_t key, int64_t i, int j) {
    const uint64_t c = 2ull * static_cast<uint64_t>(i * kTsR + j) + 1ull;
    const uint64_t w1 = splitmix_finalize(key + c * kGolden);
    const uint64_t w2 = splitmix_finalize(key + (c + 1ull) * kGolden);
    const double u1 = (static_cast<double>(w1 >> 11) + 1.0) * 0x1p-53;
    const double u2 = static_cast<double>(w2 >> 11) * 0x1p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

// Z (n x 32, fp64) and its Gram partials, one workgroup per kTsRows rows.
__global__ __launch_bounds__(256) void ts_gauss_kernel(uint64_t key, int64_t n, double *__restrict__ Z,
                                                       double *__restrict__ partials) {
    __shared__ double t[kTsRows][kTsR + 1];
    const int tid = threadIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTsRows;
    const int rows = static_cast<int>(min<int64_t>(kTsRows, n - r0));
    for (int q = tid; q < kTsRows * kTsR; q += 256) {
        const int i = q >> 5, j = q & 31;
        double z = 0.0;
        if (i < rows) {
            z = ts_gaussian(key, r0 + i, j);
            Z[(r0 + i) * kTsR + j] = z;
        }
        t[i][j] = z;
    }
    __syncthreads();
    ts_tile_gram(t, t, rows, partials + static_cast<int64_t>(blockIdx.x) * kTsGram);
}

// One workgroup: the Cholesky factor G = R^T R of the summed Gram matrix (R
// upper triangular, positive diagonal) and R^-1, fp64.
__global__ __launch_bounds__(256) void ts_chol_kernel(const double *__restrict__ gram, double *__restrict__ rinv) {
    __shared__ double g[kTsR][kTsR + 1];
    __shared__ double ri[kTsR][kTsR + 1];
    const int tid = threadIdx.x;
    for (int e = tid; e < kTsGram; e += 256) g[e >> 5][e & 31] = gram[e];
    __syncthreads();
    // right-looking, in place: row j of R in the upper triangle of row j
    for (int j = 0; j < kTsR; ++j) {
        if (tid == 0) g[j][j] = sqrt(g[j][j]);
        __syncthreads();
        const double djj = g[j][j];
        if (tid > j && tid < kTsR) g[j][tid] /= djj;
        __syncthreads();
        for (int e = tid; e < kTsGram; e += 256) {
            const int a = e >> 5, b = e & 31;
            if (a > j && b >= a) g[a][b] -= g[j][a] * g[j][b];
        }
        __syncthreads();
    }
    // column c of R^-1 by back substitution (thread c)
    if (tid < kTsR) {
        const int c = tid;
        for (int i = kTsR - 1; i >= 0; --i) {
            if (i > c) {
                ri[i][c] = 0.0;
                continue;
            }
            double s = i == c ? 1.0 : 0.0;
            for (int l = i + 1; l <= c; ++l) s -= g[i][l] * ri[l][c];
            ri[i][c] = s / g[i][i];
        }
    }
    __syncthreads();
    for (int e = tid; e < kTsGram; e += 256) rinv[e] = ri[e >> 5][e & 31];
}

// Z = Z R^-1 (fp64), one kTsRows-row block per workgroup. First pass: in
// place, with the Gram partials of the result. Second pass: the result as the
// fp32 projection P32 and its bf16 operand copy (32-row block s, column l,
// row e at element (32 s + l) 32 + e).
__global__ __launch_bounds__(256) void ts_rows_kernel(int64_t n, double *__restrict__ Z,
                                                      const double *__restrict__ rinv, double *__restrict__ partials,
                                                      float *__restrict__ P32, uint16_t *__restrict__ frag) {
    __shared__ double t[kTsRows][kTsR + 1];
    __shared__ double ri[kTsR][kTsR];
    const int tid = threadIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTsRows;
    const int rows = static_cast<int>(min<int64_t>(kTsRows, n - r0));
    for (int e = tid; e < kTsGram; e += 256) ri[e >> 5][e & 31] = rinv[e];
    for (int q = tid; q < kTsRows * kTsR; q += 256) {
        const int i = q >> 5, j = q & 31;
        t[i][j] = i < rows ? Z[(r0 + i) * kTsR + j] : 0.0;
    }
    __syncthreads();
    constexpr int kPer = kTsRows * kTsR / 256;
    double out[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int q = tid + 256 * u, i = q >> 5, j = q & 31;
        double s = 0.0;
        for (int l = 0; l <= j; ++l) s += t[i][l] * ri[l][j];
        out[u] = i < rows ? s : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int q = tid + 256 * u, i = q >> 5, j = q & 31;
        t[i][j] = out[u];
        if (i < rows) {
            if (partials)
                Z[(r0 + i) * kTsR + j] = out[u];
            else
                P32[(r0 + i) * kTsR + j] = static_cast<float>(out[u]);
        }
    }
    __syncthreads();
    if (partials) {
        ts_tile_gram(t, t, rows, partials + static_cast<int64_t>(blockIdx.x) * kTsGram);
        return;
    }
    for (int q = tid; q < kTsRows * kTsR; q += 256) {
        const int sb = q >> 10, l = (q >> 5) & 31, e = q & 31;
        const int64_t s = r0 / 32 + sb;
        if (32 * s < n) {
            // the bf16 rounding of the stored fp32 value: the float goes
            // through a register the compiler cannot see into, which keeps it
            // from folding the two roundings into one of the fp64 value
            const float x = __uint_as_float(opaque_u32(__float_as_uint(static_cast<float>(t[32 * sb + e][l]))));
            frag[(s * kTsR + l) * 32 + e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
        }
    }
}

// ------------------------------------------------------ sketch projections --

// Partial products of one 32-token block with one chunk of kTsChunkSteps
// 32-column steps: part[chunk][block][l][t] = sum over the chunk's columns c
// of A[32 block + t][c] F[c][l], F the projection (bf16 operand copy). Eight
// waves take 16 steps each; lane (i16, g) loads 8 columns of token i16 (A
// operand) and 8 rows of column i16 (B operand). grid (token blocks, chunks
// of job 0 then job 1), 512 threads.
struct TsProjJob {
    const uint16_t *A;
    int64_t lda;
    int64_t n;
    const uint16_t *frag;
    int chunks;
    int chunk0;          // first chunk of this job in the partial buffer
};
struct TsProjArgs {
    TsProjJob job[2];
    int T;
    int p_blocks;
    float *part;
};

__global__ __launch_bounds__(512) void ts_project_kernel(TsProjArgs a) {
    __shared__ __attribute__((aligned(16))) float tile[8][kTsR][32 + 4];
    const int jn = static_cast<int>(blockIdx.y) < a.job[0].chunks ? 0 : 1;
    const TsProjJob &jb = a.job[jn];
    const int chunk = static_cast<int>(blockIdx.y) - jb.chunk0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, g = lane >> 4;
    const int blk = blockIdx.x, t0 = 32 * blk;
    constexpr uint32_t kOob = 0x80000000u;   // views are below 2^31 bytes
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(jb.A), 0, static_cast<int>(static_cast<int64_t>(a.T) * jb.lda * 2), 0x00020000);
    const int nsteps = static_cast<int>((jb.n + 31) / 32);
    const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(jb.frag), 0, nsteps * kTsR * 64, 0x00020000);
    const int s_begin = min(nsteps, chunk * kTsChunkSteps + wave * (kTsChunkSteps / 8));
    const int s_end = min(nsteps, s_begin + kTsChunkSteps / 8);
    uint32_t row_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = t0 + 16 * h + i16;
        row_off[h] = t < a.T ? static_cast<uint32_t>(static_cast<int64_t>(t) * jb.lda * 2) : kOob;
    }
    auto aload = [&](int s, int h) -> u32x4_t {
        const uint32_t off = (row_off[h] != kOob && s < s_end) ? row_off[h] + static_cast<uint32_t>(2 * (32 * s + 8 * g))
                                                               : kOob;
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rs, off, 0, 0));
    };
    auto bload = [&](int s, int cb) -> u32x4_t {
        const uint32_t off = s < s_end ? static_cast<uint32_t>(((s * kTsR + 16 * cb + i16) * 32 + 8 * g) * 2) : kOob;
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rs, off, 0, 0));
    };
    f32x4_t acc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[h][cb] = zero_f32x4();
    constexpr int PF = 4;
    u32x4_t ra[PF][2], rb[PF][2];
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ra[p][h] = aload(s_begin + p, h);
            rb[p][h] = bload(s_begin + p, h);
        }
    for (int s0 = s_begin; s0 < s_end; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) acc[h][cb] = mfma_bf16(ra[p][h], rb[p][cb], acc[h][cb]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ra[p][h] = aload(s0 + p + PF, h);
                rb[p][h] = bload(s0 + p + PF, h);
            }
        }
    }
    // lane (i16, g) of (h, cb) holds tokens 16 h + 4 g + e of column 16 cb + i16
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[wave][16 * cb + i16][16 * h + 4 * g + e] = acc[h][cb][e];
    __syncthreads();
    if (tid < 256) {
        const int l = tid >> 3, q = tid & 7;
        f32x4_t s = *reinterpret_cast<const f32x4_t *>(&tile[0][l][4 * q]);
#pragma unroll
        for (int w = 1; w < 8; ++w) s += *reinterpret_cast<const f32x4_t *>(&tile[w][l][4 * q]);
        const int64_t o = ((static_cast<int64_t>(blockIdx.y) * a.p_blocks + blk) * kTsR + l) * 32 + 4 * q;
        *reinterpret_cast<f32x4_t *>(a.part + o) = s;
    }
}

// out_j = bf16(sum over job j's chunks, in chunk order, of the partials);
// 8 elements per thread, grid (ceil(elems / 2048), 2). The first workgroup
// also zeroes the sync words of the two folds that follow.
struct TsProjReduceArgs {
    const float *part;
    int chunks[2];
    int chunk0[2];
    int64_t elems;          // p_blocks * 32 * 32
    uint16_t *out[2];
    int *sync[2];
    int n_sync[2];
};

__global__ __launch_bounds__(256) void ts_project_reduce_kernel(TsProjReduceArgs a) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && blockIdx.y == 0) {
        for (int f = 0; f < 2; ++f)
            for (int i = tid; i < a.n_sync[f]; i += 256) a.sync[f][i] = 0;
    }
    const int j = blockIdx.y;
    const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 256 + tid) * 8;
    if (idx >= a.elems) return;
    const float *p = a.part + static_cast<int64_t>(a.chunk0[j]) * a.elems + idx;
    f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p), hi = *reinterpret_cast<const f32x4_t *>(p + 4);
    for (int c = 1; c < a.chunks[j]; ++c) {
        lo += *reinterpret_cast<const f32x4_t *>(p + c * a.elems);
        hi += *reinterpret_cast<const f32x4_t *>(p + c * a.elems + 4);
    }
    *reinterpret_cast<u32x4_t *>(a.out[j] + idx) =
        u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
}

// ----------------------------------------------------------------- update --

// Moments and normalized sketch of one kTsRows-row block of S_R (blocks
// 0 .. nr - 1) or of S_L^T (blocks nr ..), with its fp64 Gram partials in two
// 1024-double slots per block: slot 0 the Gram matrix of the block of U,
// slot 1 (S_R blocks only) the block's part of P^T U_R.
struct TsUpdateArgs {
    const float *S_L, *S_R;     // k x 32, d x 32
    const float *P;             // d x 32 (fp32)
    float *m_L, *v_L, *m_R, *v_R;
    float *U_L, *U_R;           // k x 32, d x 32
    double *partials;
    int64_t d, k;
    int nr;
    float beta1, beta2, eps;
};

__global__ __launch_bounds__(256) void ts_moments_kernel(TsUpdateArgs a) {
    __shared__ float u[kTsRows][kTsR + 1];
    __shared__ float p[kTsRows][kTsR + 1];
    const int tid = threadIdx.x;
    const bool right = static_cast<int>(blockIdx.x) < a.nr;
    const int blk = right ? static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x) - a.nr;
    const int64_t n = right ? a.d : a.k;
    const float *S = right ? a.S_R : a.S_L;
    float *m = right ? a.m_R : a.m_L;
    float *v = right ? a.v_R : a.v_L;
    float *U = right ? a.U_R : a.U_L;
    const int64_t r0 = static_cast<int64_t>(blk) * kTsRows;
    const int rows = static_cast<int>(min<int64_t>(kTsRows, n - r0));
    for (int q = tid; q < kTsRows * kTsR; q += 256) {
        const int i = q >> 5, j = q & 31;
        float uu = 0.f, pp = 0.f;
        if (i < rows) {
            const int64_t x = (r0 + i) * kTsR + j;
            const float s = S[x];
            const float mn = a.beta1 * m[x] + (1.f - a.beta1) * s;
            const float vn = a.beta2 * v[x] + (1.f - a.beta2) * (s * s);
            m[x] = mn;
            v[x] = vn;
            uu = mn / (sqrtf(vn) + a.eps);
            U[x] = uu;
            if (right) pp = a.P[x];
        }
        u[i][j] = uu;
        p[i][j] = pp;
    }
    __syncthreads();
    double *out = a.partials + static_cast<int64_t>(blockIdx.x) * 2 * kTsGram;
    ts_tile_gram(u, u, rows, out);
    if (right) ts_tile_gram(p, u, rows, out + kTsGram);
}

// Round `round` of the circle schedule over 32 indices: pair k of 16
// (index 0 fixed, the other 31 on a ring); every pair of indices meets once
// in 31 rounds, and the 16 pairs of a round cover all 32 indices.
__device__ __forceinline__ void ts_pair(int round, int k, int &p, int &q) {
    if (k == 0) {
        p = 0;
        q = round % 31 + 1;
    } else {
        p = (round + k) % 31 + 1;
        q = (round - k + 31) % 31 + 1;
    }
    if (p > q) {
        const int x = p;
        p = q;
        q = x;
    }
}

constexpr int kTsMaxSweeps = 40;

// 1 / sqrt(x) and 1 / x for finite x > 0 (x != 0): the hardware estimates
// refined by two Newton steps each (the estimates hold about half the fp64
// bits; each step doubles them), short dependent chains where the library's
// correctly rounded sqrt and division are long ones.
__device__ __forceinline__ double ts_rsqrt(double x) {
    double y = __builtin_amdgcn_rsq(x);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double e = fma(-x * y, y, 1.0);
        y = fma(0.5 * y, e, y);
    }
    return y;
}
__device__ __forceinline__ double ts_rcp(double x) {
    double y = __builtin_amdgcn_rcp(x);
#pragma unroll
    for (int i = 0; i < 2; ++i) y = fma(y, fma(-x, y, 1.0), y);
    return y;
}

// Whether the Jacobi rotation of a pair with diagonal entries al, be and
// off-diagonal entry ga is due: |ga| above 1e-15 sqrt(|al be|) and above
// `floor_abs` (the level of fp64 rounding in H); false for non-finite input.
__device__ __forceinline__ bool ts_rotation_due(double al, double be, double ga, double floor_abs) {
    return ga * ga > 1e-30 * fabs(al * be) && fabs(ga) > floor_abs;
}

// The rotation that zeroes ga: column p' = c col_p - s col_q,
// q' = s col_p + c col_q, with t = s / c the smaller root (Rutishauser's
// form); the identity (c = 1, s = t = 0) when it is not due. Computed without
// branches, so that the rotations of a thread's two pairs overlap.
__device__ __forceinline__ bool ts_rotation(double al, double be, double ga, double floor_abs, double &c, double &s,
                                            double &t) {
    const bool due = ts_rotation_due(al, be, ga, floor_abs);
    const double d = be - al, g2 = 2.0 * ga;
    const double sq = fma(d, d, g2 * g2);
    const double r = sq * ts_rsqrt(sq);
    const double tt = g2 * ts_rcp(d >= 0.0 ? d + r : d - r);
    const double cc = ts_rsqrt(fma(tt, tt, 1.0));
    c = due ? cc : 1.0;
    s = due ? cc * tt : 0.0;
    t = due ? tt : 0.0;
    return due;
}

// Sum over the 32 lanes of a half-wave by a butterfly of lane exchanges:
// DPP quad swaps (lane ^ 1, lane ^ 2), the half-row and row mirrors (lane i
// with 7 - i, then 15 - i: after the quad sums these pair up disjoint halves
// just as xor 4 and xor 8 would) and a swizzle that swaps the two 16-lane
// rows. Each stage adds two partial sums that are each other's mirror image
// and fp64 addition commutes, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ double ts_dpp(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF,
                                               true);
    return __longlong_as_double(static_cast<long long>(
        (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo)));
}
__device__ __forceinline__ double ts_swap16(double x) {
    // bit-mask swizzle within 32 lanes: and 0x1F, or 0, xor 0x10
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const int lo = __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(u)), 0x401F);
    const int hi = __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(u >> 32)), 0x401F);
    return __longlong_as_double(static_cast<long long>(
        (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo)));
}
__device__ __forceinline__ double ts_half_wave_sum(double x) {
    x += ts_dpp<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += ts_dpp<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += ts_dpp<0x141>(x);   // row_half_mirror
    x += ts_dpp<0x140>(x);   // row_mirror
    x += ts_swap16(x);
    return x;
}

constexpr int kTsCoupleThreads = 512;   // 16 column pairs x 32 rows

// One workgroup of 512 threads. sums: [U_R^T U_R][P^T U_R][U_L U_L^T] (1024
// doubles each). The pseudo-inverse of M = P^T U_R by one-sided Jacobi on
// its columns (fp64): A = M V converges to U Sigma, so the singular values
// are A's column norms and C = V Sigma^+ U^T = sum_j v_j a_j^T / sigma_j^2
// over the kept j (singular values at most 32 2^-23 times the largest count
// as zero). A and V live in LDS column by column. A round rotates 16
// disjoint column pairs at once: thread (pair, row) reads its row's entries
// of the pair's two columns of A and of V, the pair's 32 threads (one
// half-wave) add the three dot products by a butterfly, each computes the
// same rotation and writes its four rotated entries back; one barrier per
// round. The loop ends after a sweep in which no pair was due. Writes C
// (fp32) and sqnorm = ||U_R C U_L||_F^2 (from the Gram matrices of U_R and
// U_L, fp64).
__global__ __launch_bounds__(kTsCoupleThreads) void ts_couple_kernel(const double *__restrict__ sums,
                                                                     float *__restrict__ C_out,
                                                                     float *__restrict__ sqnorm) {
    __shared__ double A[kTsR][kTsR];          // A[col][row]
    __shared__ double V[kTsR][kTsR];          // V[col][row]
    __shared__ double GR[kTsR][kTsR + 1];
    __shared__ double GL[kTsR][kTsR + 1];
    __shared__ double Cm[kTsR][kTsR + 1];
    __shared__ double X[kTsR][kTsR + 1];
    __shared__ double norm2[kTsR];
    __shared__ double inv[kTsR];
    __shared__ double red[kTsCoupleThreads];
    __shared__ int s_flag[3];
    const int tid = threadIdx.x;
    for (int e = tid; e < kTsGram; e += kTsCoupleThreads) {
        const int i = e >> 5, j = e & 31;
        GR[i][j] = sums[e];
        A[j][i] = sums[kTsGram + e];          // M[i][j]
        GL[i][j] = sums[2 * kTsGram + e];
        V[j][i] = i == j ? 1.0 : 0.0;
    }
    if (tid < 3) s_flag[tid] = 0;
    __syncthreads();
    // ||M||_F^2, the scale of fp64 rounding in the dot products
    if (tid < kTsR) {
        double s2 = 0.0;
        for (int i = 0; i < kTsR; ++i) s2 += A[tid][i] * A[tid][i];
        norm2[tid] = s2;
    }
    __syncthreads();
    double tr = 0.0;
    for (int j = 0; j < kTsR; ++j) tr += norm2[j];
    const double floor_abs = 0x1p-52 * tr / kTsR;
    const int k = tid >> 5, row = tid & 31;
    for (int sweep = 0; sweep < kTsMaxSweeps; ++sweep) {
        if (tid == 0) s_flag[(sweep + 1) % 3] = 0;
        for (int round = 0; round < 31; ++round) {
            int p, q;
            ts_pair(round, k, p, q);
            const double ap = A[p][row], aq = A[q][row], vp = V[p][row], vq = V[q][row];
            const double al = ts_half_wave_sum(ap * ap);
            const double be = ts_half_wave_sum(aq * aq);
            const double ga = ts_half_wave_sum(ap * aq);
            double c, sn, t;
            if (ts_rotation(al, be, ga, floor_abs, c, sn, t) && row == 0) s_flag[sweep % 3] = 1;
            A[p][row] = c * ap - sn * aq;
            A[q][row] = sn * ap + c * aq;
            V[p][row] = c * vp - sn * vq;
            V[q][row] = sn * vp + c * vq;
            __syncthreads();
        }
        // converged once a whole sweep found no pair due
        if (s_flag[sweep % 3] == 0) break;
    }
    // singular values (column norms of A), the cutoff and 1 / sigma^2
    if (tid < kTsR) {
        double s2 = 0.0;
        for (int i = 0; i < kTsR; ++i) s2 += A[tid][i] * A[tid][i];
        norm2[tid] = s2;
    }
    __syncthreads();
    if (tid < kTsR) {
        double smax = 0.0;
        for (int j = 0; j < kTsR; ++j) smax = fmax(smax, sqrt(norm2[j]));
        inv[tid] = sqrt(norm2[tid]) > 32.0 * 0x1p-23 * smax ? 1.0 / norm2[tid] : 0.0;
    }
    __syncthreads();
    // C[a][b] = sum_j V[a][j] A[b][j] / sigma_j^2
    for (int e = tid; e < kTsGram; e += kTsCoupleThreads) {
        const int a = e >> 5, b = e & 31;
        double c = 0.0;
        for (int j = 0; j < kTsR; ++j) c += V[j][a] * (inv[j] * A[j][b]);
        Cm[a][b] = c;
        C_out[e] = static_cast<float>(c);
    }
    __syncthreads();
    // sqnorm = sum (C^T GR C) o GL, with X = GR C
    for (int e = tid; e < kTsGram; e += kTsCoupleThreads) {
        const int i = e >> 5, j = e & 31;
        double x = 0.0;
        for (int l = 0; l < kTsR; ++l) x += GR[i][l] * Cm[l][j];
        X[i][j] = x;
    }
    __syncthreads();
    double part = 0.0;
    for (int e = tid; e < kTsGram; e += kTsCoupleThreads) {
        const int i = e >> 5, j = e & 31;
        double x = 0.0;
        for (int l = 0; l < kTsR; ++l) x += Cm[l][i] * X[l][j];
        part += x * GL[i][j];
    }
    red[tid] = part;
    __syncthreads();
    for (int w = kTsCoupleThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) sqnorm[0] = static_cast<float>(red[0]);
}

// B = U_R C (d x 32, fp32): four threads per row, eight columns each.
__global__ __launch_bounds__(256) void ts_b_kernel(const float *__restrict__ U_R, const float *__restrict__ C,
                                                   int64_t d, float *__restrict__ Bm) {
    __shared__ float c[kTsR][kTsR];
    const int tid = threadIdx.x;
    for (int e = tid; e < kTsGram; e += 256) c[e >> 5][e & 31] = C[e];
    __syncthreads();
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 64 + (tid >> 2);
    const int c0 = 8 * (tid & 3);
    if (row >= d) return;
    float u[kTsR];
#pragma unroll
    for (int e = 0; e < kTsR; e += 4) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(U_R + row * kTsR + e);
        u[e] = x.x;
        u[e + 1] = x.y;
        u[e + 2] = x.z;
        u[e + 3] = x.w;
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < kTsR; ++e) s = fmaf(u[e], c[e][c0 + j], s);
        o[j] = s;
    }
    *reinterpret_cast<f32x4_t *>(Bm + row * kTsR + c0) = f32x4_t{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4_t *>(Bm + row * kTsR + c0 + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
}

// ------------------------------------------------------------------ apply --

// Eight fp32 values -> a bf16 head (round to nearest) and the bf16 of what
// the head leaves over.
__device__ __forceinline__ void ts_split8(const float *src, u32x4_t &head, u32x4_t &tail) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(src);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(src + 4);
    const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t h[4], t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        h[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
        t[q] = pack_bf16x2(x[2 * q] - bf16_lo(h[q]), x[2 * q + 1] - bf16_hi(h[q]));
    }
    head = u32x4_t{h[0], h[1], h[2], h[3]};
    tail = u32x4_t{t[0], t[1], t[2], t[3]};
}

// W -= step B U_L over a 128 x 128 tile: four waves of 64 x 64, three
// 16x16x32 products per 16 x 16 block (the rank is the contraction); the tile
// goes through LDS (fp32) and W moves in 16-byte pieces of rows.
template <bool WBF16>
__global__ __launch_bounds__(256) void ts_apply_kernel(const float *__restrict__ Bm, const float *__restrict__ U_L,
                                                       int64_t d, int64_t k, void *__restrict__ W, int64_t ldw,
                                                       float step) {
    __shared__ __attribute__((aligned(16))) float tile[128][128 + 4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int i16 = lane & 15, g = lane >> 4;
    const int64_t row0 = static_cast<int64_t>(blockIdx.y) * 128, col0 = static_cast<int64_t>(blockIdx.x) * 128;
    u32x4_t ah[4], at[4], bh[4], bt[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int64_t r = row0 + 64 * wm + 16 * mb + i16;
        if (r < d) {
            ts_split8(Bm + r * kTsR + 8 * g, ah[mb], at[mb]);
        } else {
            ah[mb] = zero_u32x4();
            at[mb] = zero_u32x4();
        }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t c = col0 + 64 * wn + 16 * nb + i16;
        if (c < k) {
            ts_split8(U_L + c * kTsR + 8 * g, bh[nb], bt[nb]);
        } else {
            bh[nb] = zero_u32x4();
            bt[nb] = zero_u32x4();
        }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            // lane (i16, g) holds rows 4 g + e of column i16 of the block
            f32x4_t acc = mfma_bf16(at[mb], bh[nb], zero_f32x4());
            acc = mfma_bf16(ah[mb], bt[nb], acc);
            acc = mfma_bf16(ah[mb], bh[nb], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[64 * wm + 16 * mb + 4 * g + e][64 * wn + 16 * nb + i16] = acc[e];
        }
    __syncthreads();
    constexpr int EPC = WBF16 ? 8 : 4;   // elements per 16-byte piece
    constexpr int PPR = 128 / EPC;       // pieces per tile row
    for (int q = tid; q < 128 * PPR; q += 256) {
        const int r = q / PPR, c = (q - r * PPR) * EPC;
        const int64_t row = row0 + r, col = col0 + c;
        if (row >= d || col >= k) continue;
        if (WBF16) {
            uint16_t *wp = static_cast<uint16_t *>(W) + row * ldw + col;
            const u32x4_t wv = *reinterpret_cast<const u32x4_t *>(wp);
            uint32_t o[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = fmaf(-step, tile[r][c + 2 * h], bf16_lo(wv[h]));
                const float hi = fmaf(-step, tile[r][c + 2 * h + 1], bf16_hi(wv[h]));
                o[h] = pack_bf16x2(lo, hi);
            }
            *reinterpret_cast<u32x4_t *>(wp) = u32x4_t{o[0], o[1], o[2], o[3]};
        } else {
            float *wp = static_cast<float *>(W) + row * ldw + col;
            f32x4_t wv = *reinterpret_cast<const f32x4_t *>(wp);
#pragma unroll
            for (int h = 0; h < 4; ++h) wv[h] = fmaf(-step, tile[r][c + h], wv[h]);
            *reinterpret_cast<f32x4_t *>(wp) = wv;
        }
    }
}

// ---------------------------------------------------------------- launchers --

TsProjLayout ts_projection_layout(int64_t n) {
    TsProjLayout L;
    L.n_blocks = static_cast<int>((n + kTsRows - 1) / kTsRows);
    L.fp32_bytes = align256(static_cast<size_t>(n) * kTsR * 4);
    L.frag_bytes = align256(static_cast<size_t>((n + 31) / 32) * 32 * kTsR * 2);
    L.z_bytes = align256(static_cast<size_t>(n) * kTsR * 8);
    L.partial_bytes = align256(static_cast<size_t>(L.n_blocks) * kTsGram * 8);
    L.gram_bytes = align256(kTsGram * 8);
    L.rinv_bytes = align256(kTsGram * 8);
    L.total = L.fp32_bytes + L.frag_bytes + L.z_bytes + L.partial_bytes + L.gram_bytes + L.rinv_bytes;
    return L;
}

hipError_t launch_ts_projection(uint64_t key, int64_t n, void *buf, hipStream_t st) {
    const TsProjLayout L = ts_projection_layout(n);
    char *p = static_cast<char *>(buf);
    float *P32 = reinterpret_cast<float *>(p);
    p += L.fp32_bytes;
    uint16_t *frag = reinterpret_cast<uint16_t *>(p);
    p += L.frag_bytes;
    double *Z = reinterpret_cast<double *>(p);
    p += L.z_bytes;
    double *partials = reinterpret_cast<double *>(p);
    p += L.partial_bytes;
    double *gram = reinterpret_cast<double *>(p);
    p += L.gram_bytes;
    double *rinv = reinterpret_cast<double *>(p);
    TsSumArgs sa{};
    sa.job[0] = TsSumJob{partials, kTsGram, 0, L.n_blocks, gram};
    hipLaunchKernelGGL(ts_gauss_kernel, dim3(L.n_blocks), dim3(256), 0, st, key, n, Z, partials);
    for (int pass = 0; pass < 2; ++pass) {
        hipError_t e = launch_sum(sa, 1, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(ts_chol_kernel, dim3(1), dim3(256), 0, st, gram, rinv);
        hipLaunchKernelGGL(ts_rows_kernel, dim3(L.n_blocks), dim3(256), 0, st, n, Z, rinv,
                           pass == 0 ? partials : nullptr, P32, frag);
    }
    return hipGetLastError();
}

TsSketchLayout ts_sketch_layout(int64_t T, int64_t d, int64_t k) {
    TsSketchLayout L;
    L.p_blocks = static_cast<int>((T + 31) / 32);
    L.chunks[0] = static_cast<int>(((k + 31) / 32 + kTsChunkSteps - 1) / kTsChunkSteps);
    L.chunks[1] = static_cast<int>(((d + 31) / 32 + kTsChunkSteps - 1) / kTsChunkSteps);
    L.p_bytes = align256(static_cast<size_t>(L.p_blocks) * 32 * kTsR * 2);
    L.part_bytes = align256(static_cast<size_t>(L.chunks[0] + L.chunks[1]) * L.p_blocks * 32 * kTsR * 4);
    L.fold[0] = plan_fold_bf16(T, d, kTsR);
    L.fold[1] = plan_fold_bf16(T, k, kTsR);
    L.fold_off[0] = 2 * L.p_bytes + L.part_bytes;
    L.fold_off[1] = L.fold_off[0] + L.fold[0].xbuf_bytes + L.fold[0].sync_bytes;
    L.total = L.fold_off[1] + L.fold[1].xbuf_bytes + L.fold[1].sync_bytes;
    return L;
}

hipError_t launch_ts_sketch(int64_t T, int64_t d, int64_t k, const uint16_t *X, int64_t ldx, const uint16_t *dY,
                            int64_t lddy, const void *projP, const void *projQ, float *S_L, float *S_R,
                            int accumulate, void *ws, const FoldWait &wait, hipStream_t st) {
    const TsSketchLayout L = ts_sketch_layout(T, d, k);
    char *base = static_cast<char *>(ws);
    uint16_t *Xq = reinterpret_cast<uint16_t *>(base);
    uint16_t *Yp = reinterpret_cast<uint16_t *>(base + L.p_bytes);
    float *part = reinterpret_cast<float *>(base + 2 * L.p_bytes);
    const TsProjLayout LP = ts_projection_layout(d), LQ = ts_projection_layout(k);
    const uint16_t *fragQ = reinterpret_cast<const uint16_t *>(static_cast<const char *>(projQ) + LQ.fp32_bytes);
    const uint16_t *fragP = reinterpret_cast<const uint16_t *>(static_cast<const char *>(projP) + LP.fp32_bytes);
    TsProjArgs a;
    a.job[0] = TsProjJob{X, ldx, k, fragQ, L.chunks[0], 0};
    a.job[1] = TsProjJob{dY, lddy, d, fragP, L.chunks[1], L.chunks[0]};
    a.T = static_cast<int>(T);
    a.p_blocks = L.p_blocks;
    a.part = part;
    hipLaunchKernelGGL(ts_project_kernel, dim3(L.p_blocks, L.chunks[0] + L.chunks[1]), dim3(512), 0, st, a);
    TsProjReduceArgs r;
    r.part = part;
    r.chunks[0] = L.chunks[0];
    r.chunks[1] = L.chunks[1];
    r.chunk0[0] = 0;
    r.chunk0[1] = L.chunks[0];
    r.elems = static_cast<int64_t>(L.p_blocks) * 32 * kTsR;
    r.out[0] = Xq;
    r.out[1] = Yp;
    for (int f = 0; f < 2; ++f) {
        r.sync[f] = reinterpret_cast<int *>(base + L.fold_off[f] + L.fold[f].xbuf_bytes);
        r.n_sync[f] = L.fold[f].sync_words;
    }
    hipLaunchKernelGGL(ts_project_reduce_kernel, dim3(static_cast<unsigned>((r.elems / 8 + 255) / 256), 2),
                       dim3(256), 0, st, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // S_R (+)= dY^T Xq (d x 32), then S_L^T (+)= X^T Yp (k x 32)
    e = launch_fold_bf16_tiles(kTsR, T, d, dY, lddy, Xq, L.p_blocks, S_R, accumulate, base + L.fold_off[0], wait,
                               st);
    if (e != hipSuccess) return e;
    return launch_fold_bf16_tiles(kTsR, T, k, X, ldx, Yp, L.p_blocks, S_L, accumulate, base + L.fold_off[1], wait,
                                  st);
}

TsUpdateLayout ts_update_layout(int64_t d, int64_t k) {
    TsUpdateLayout L;
    L.nr = static_cast<int>((d + kTsRows - 1) / kTsRows);
    L.nl = static_cast<int>((k + kTsRows - 1) / kTsRows);
    L.ur_off = 0;
    L.ul_off = L.ur_off + align256(static_cast<size_t>(d) * kTsR * 4);
    L.b_off = L.ul_off + align256(static_cast<size_t>(k) * kTsR * 4);
    L.c_off = L.b_off + align256(static_cast<size_t>(d) * kTsR * 4);
    L.sums_off = L.c_off + align256(kTsGram * 4);
    L.partial_off = L.sums_off + align256(3 * kTsGram * 8);
    L.total = L.partial_off + align256(static_cast<size_t>(L.nr + L.nl) * 2 * kTsGram * 8);
    return L;
}

hipError_t launch_ts_update(int64_t d, int64_t k, const float *S_L, const float *S_R, const void *projP, float *m_L,
                            float *v_L, float *m_R, float *v_R, float beta1, float beta2, float eps, float *sqnorm,
                            void *ws, hipStream_t st) {
    const TsUpdateLayout L = ts_update_layout(d, k);
    char *base = static_cast<char *>(ws);
    TsUpdateArgs a;
    a.S_L = S_L;
    a.S_R = S_R;
    a.P = static_cast<const float *>(projP);
    a.m_L = m_L;
    a.v_L = v_L;
    a.m_R = m_R;
    a.v_R = v_R;
    a.U_R = reinterpret_cast<float *>(base + L.ur_off);
    a.U_L = reinterpret_cast<float *>(base + L.ul_off);
    a.partials = reinterpret_cast<double *>(base + L.partial_off);
    a.d = d;
    a.k = k;
    a.nr = L.nr;
    a.beta1 = beta1;
    a.beta2 = beta2;
    a.eps = eps;
    float *Bm = reinterpret_cast<float *>(base + L.b_off);
    float *C = reinterpret_cast<float *>(base + L.c_off);
    double *sums = reinterpret_cast<double *>(base + L.sums_off);
    hipLaunchKernelGGL(ts_moments_kernel, dim3(L.nr + L.nl), dim3(256), 0, st, a);
    TsSumArgs sa;
    sa.job[0] = TsSumJob{a.partials, 2 * kTsGram, 0, L.nr, sums};
    sa.job[1] = TsSumJob{a.partials + kTsGram, 2 * kTsGram, 0, L.nr, sums + kTsGram};
    sa.job[2] = TsSumJob{a.partials, 2 * kTsGram, L.nr, L.nl, sums + 2 * kTsGram};
    hipError_t e = launch_sum(sa, 3, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ts_couple_kernel, dim3(1), dim3(kTsCoupleThreads), 0, st, sums, C, sqnorm);
    hipLaunchKernelGGL(ts_b_kernel, dim3(static_cast<unsigned>((d + 63) / 64)), dim3(256), 0, st, a.U_R, C, d, Bm);
    return hipGetLastError();
}

hipError_t launch_ts_apply(int64_t d, int64_t k, const void *ws, void *W, int w_bf16, int64_t ldw, float step,
                           hipStream_t st) {
    const TsUpdateLayout L = ts_update_layout(d, k);
    const char *base = static_cast<const char *>(ws);
    const float *U_L = reinterpret_cast<const float *>(base + L.ul_off);
    const float *Bm = reinterpret_cast<const float *>(base + L.b_off);
    const dim3 grid(static_cast<unsigned>((k + 127) / 128), static_cast<unsigned>((d + 127) / 128));
    if (w_bf16)
        hipLaunchKernelGGL(ts_apply_kernel<true>, grid, dim3(256), 0, st, Bm, U_L, d, k, W, ldw, step);
    else
        hipLaunchKernelGGL(ts_apply_kernel<false>, grid, dim3(256), 0, st, Bm, U_L, d, k, W, ldw, step);
    return hipGetLastError();
}

}  // namespace logra
