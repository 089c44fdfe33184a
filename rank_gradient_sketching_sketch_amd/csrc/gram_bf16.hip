// Apply pass 1 for bf16 compute: the per-row sums of squares of Ghat = S A
// and the step controller's reduction, from the r x r Gram matrix of the
// signs instead of a d x k reconstruction.
//
// RowAdam keeps one second moment per row ("NVIDIA's LoGRA fits RL
// post-training of a 27B model onto a single eight-GPU node", sections "What
// happened" and "Why it matters"); pass 1 needs rowsq_i = sum_j Ghat_ij^2 for
// it and the controller needs sum_i rowsq_i / (sqrt(v'_i) + eps)^2 ("LoGRA:
// Scaling LLM Reinforcement Learning...", paragraph "Step control."). With
// A = c Sigma,
//     rowsq_i = ||S_i A||^2 = c^2 S_i (Sigma Sigma^T) S_i^T = c^2 S_i M S_i^T,
// the same number up to rounding, for 2 r^2 (d + k) operations instead of
// 2 d k r. M_lm = k - 2 popcount(sigma_l xor sigma_m) is an exact integer
// (column tail masked). The diagonal part k ||S_i||^2 is summed in fp32; the
// off-diagonal part Y = S M_off runs on bf16 MFMA (S rounded to bf16 as in
// pass 2; M_off rounded to bf16, exact for |M_lm| <= 256) and is dotted with
// the fp32 S row.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

// M_off[l][m] (bf16, row-major r x r, zero diagonal) = k - 2 popcount(sigma_l
// xor sigma_m). A workgroup owns a 16 x 16 tile of (l, m); the sign words of
// its 32 rows are hashed into LDS 64 blocks at a time (rows padded by one
// word so the 16 rows of a column read fall on different banks) and each
// thread counts the sign differences of its pair.
constexpr int kGramChunk = 64;   // 64-bit words per row per chunk

__global__ __launch_bounds__(256) void gram_kernel(uint64_t key, int R, int K, uint16_t *__restrict__ M) {
    __shared__ uint64_t wl[16][kGramChunk + 1];
    __shared__ uint64_t wm[16][kGramChunk + 1];
    const int tid = threadIdx.x;
    const int l0 = blockIdx.y * 16, m0 = blockIdx.x * 16;
    const int tl = tid >> 4, tm = tid & 15;
    const int nb = (K + 63) / 64;
    const int tail = K - 64 * (nb - 1);
    const uint64_t last_mask = tail == 64 ? ~0ull : ((1ull << tail) - 1ull);
    int pc = 0;
    for (int b0 = 0; b0 < nb; b0 += kGramChunk) {
        const int bn = min(kGramChunk, nb - b0);
        for (int idx = tid; idx < 2 * 16 * kGramChunk; idx += 256) {
            const int which = idx / (16 * kGramChunk);
            const int rem = idx - which * 16 * kGramChunk;
            const int row = rem / kGramChunk, bb = rem - row * kGramChunk;
            uint64_t w = 0;
            if (bb < bn) {
                w = sign_word(key, static_cast<uint32_t>((which ? m0 : l0) + row), static_cast<uint32_t>(b0 + bb));
                if (b0 + bb == nb - 1) w &= last_mask;   // columns past k do not count
            }
            (which ? wm : wl)[row][bb] = w;
        }
        __syncthreads();
        for (int bb = 0; bb < bn; ++bb) pc += __popcll(wl[tl][bb] ^ wm[tm][bb]);
        __syncthreads();
    }
    const int l = l0 + tl, m = m0 + tm;
    const float v = l == m ? 0.f : static_cast<float>(K - 2 * pc);
    M[static_cast<size_t>(l) * R + m] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// rowsq_i = c^2 (k ||S_i||^2 + sum_m S_im Y_im), Y^T = M_off S^T. A workgroup
// owns 128 rows of S, one wave 32 of them (two 16-row blocks i). M_off is
// copied into LDS once per workgroup by direct global-to-LDS loads (no
// registers), with the 16-byte chunks of row r stored in the order
// chunk ^ (r mod 16), so a fragment's 16 rows fall on different banks.
// The MFMA forms 16 x 16 blocks of Y^T with A = rows of M_off (LDS) and
// B = S^T (bf16, registers). Row r = 4 q + e of block mb stands for
// m = 32 (mb / 2) + 8 q + 4 (mb % 2) + e (M_off is symmetric, so any order of
// m is a valid A operand), which puts in lane (n, g) exactly the Y[i][m] whose
// S[i][m] it already holds in fp32 for its B fragment: the dot product and
// the squares need no further loads.
template <int R>
__global__ __launch_bounds__(256) void rowsq_gram_kernel(const float *__restrict__ S, int D, int K,
                                                         const uint16_t *__restrict__ M, float c,
                                                         const float *__restrict__ v, float beta2,
                                                         float eps, float *__restrict__ rowsq,
                                                         float *__restrict__ partials) {
    constexpr int KS = R / 32;                 // 32-wide steps of the rank
    constexpr int NB = R / 16;                 // 16-row blocks of m
    constexpr int CPR = R / 8;                 // 16-byte chunks per row of M_off
    constexpr int SW = CPR < 16 ? CPR : 16;    // chunk swizzle period
    __shared__ __attribute__((aligned(16))) uint16_t ms[R * R];
    __shared__ float terms[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int i0 = blockIdx.x * 128 + wave * 32;

    // This lane's S values, issued first: row i0 + 16 ib + n, columns
    // 32 s + 8 g .. +7 (the B fragment before rounding, and the entries its
    // Y values meet).
    f32x4_t raw[2][KS][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const float *srow = S + static_cast<int64_t>(min(i0 + 16 * ib + n, D - 1)) * R;   // rows past d are dropped
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            raw[ib][s][0] = *reinterpret_cast<const f32x4_t *>(srow + 32 * s + 8 * g);
            raw[ib][s][1] = *reinterpret_cast<const f32x4_t *>(srow + 32 * s + 8 * g + 4);
        }
    }
    // stage M_off: each wave instruction moves 64 chunks; lane i's chunk
    // lands at LDS chunk position q0 + i (row q / CPR, position q % CPR) and
    // carries logical chunk position ^ (row mod SW)
    for (int q0 = wave * 64; q0 < R * CPR; q0 += 256) {
        const int q = q0 + lane;
        const int row = q / CPR, pos = q - row * CPR;
        const int ch = pos ^ (row & (SW - 1));
        __builtin_amdgcn_global_load_lds(M + static_cast<size_t>(row) * R + 8 * ch,
                                         (__attribute__((address_space(3))) void *)(ms + q0 * 8), 16, 0, 0);
    }
    u32x4_t bt[2][KS];
    float ssq[2] = {0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const f32x4_t lo = raw[ib][s][0], hi = raw[ib][s][1];
            bt[ib][s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                                pack_bf16x2(hi.z, hi.w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) ssq[ib] = fmaf(hi[e], hi[e], fmaf(lo[e], lo[e], ssq[ib]));
        }
    __syncthreads();

    // A row n of block mb: m = 32 (mb / 2) + 8 (n / 4) + 4 (mb % 2) + n % 4
    const int mrow_base = 8 * (n >> 2) + (n & 3);
    float ydot[2] = {0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
        const int mrow = 32 * (mb >> 1) + 4 * (mb & 1) + mrow_base;
        f32x4_t acc[2] = {zero_f32x4(), zero_f32x4()};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4_t af =
                *reinterpret_cast<const u32x4_t *>(&ms[mrow * R + 8 * ((4 * s + g) ^ (mrow & (SW - 1)))]);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) acc[ib] = mfma_bf16(af, bt[ib][s], acc[ib]);
        }
        // lane (n, g) now holds Y[i][32 (mb / 2) + 8 g + 4 (mb % 2) + e]
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const f32x4_t sv = raw[ib][mb >> 1][mb & 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) ydot[ib] = fmaf(sv[e], acc[ib][e], ydot[ib]);
        }
    }
    // add the four lanes of a row (g = 0..3), fixed butterfly order
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            ydot[ib] += __shfl_xor(ydot[ib], off, 64);
            ssq[ib] += __shfl_xor(ssq[ib], off, 64);
        }
    // lanes g == ib write row i0 + 16 ib + n
    float term = 0.f;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int i = i0 + 16 * ib + n;
        if (g == ib && i < D) {
            const float rq = (c * c) * fmaf(static_cast<float>(K), ssq[ib], ydot[ib]);
            rowsq[i] = rq;
            const float vn = beta2 * v[i] + (1.f - beta2) * (rq / static_cast<float>(K));
            const float u = 1.f / (sqrtf(vn) + eps);
            term += rq * u * u;
        }
    }
    // per-workgroup partial of the controller's reduction, fixed order
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) term += __shfl_xor(term, off, 64);
    if (lane == 0) terms[wave] = term;
    __syncthreads();
    if (tid == 0) partials[blockIdx.x] = ((terms[0] + terms[1]) + terms[2]) + terms[3];
}

SqnormPlan plan_sqnorm_bf16(int64_t D, int64_t K, int R) {
    SqnormPlan p;
    p.n_blocks = static_cast<int>((D + 127) / 128);
    (void)K;
    const size_t align = 256;
    p.partial_bytes = (static_cast<size_t>(p.n_blocks) * 4 + align - 1) / align * align;
    p.gram_bytes = (static_cast<size_t>(R) * R * 2 + align - 1) / align * align;
    return p;
}

template <int R>
static hipError_t sqnorm_r(const ApplyArgs &a, void *ws, hipStream_t st) {
    const SqnormPlan p = plan_sqnorm_bf16(a.D, a.K, R);
    char *base = static_cast<char *>(ws);
    float *partials = reinterpret_cast<float *>(base);
    uint16_t *M = reinterpret_cast<uint16_t *>(base + p.partial_bytes);
    const int K = static_cast<int>(a.K);
    hipLaunchKernelGGL(gram_kernel, dim3(R / 16, R / 16), dim3(256), 0, st, a.key, R, K, M);
    hipLaunchKernelGGL(rowsq_gram_kernel<R>, dim3(p.n_blocks), dim3(256), 0, st, a.S,
                       static_cast<int>(a.D), K, M, a.c, a.v_in, a.beta2, a.eps, a.rowsq_out, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_sqnorm_final(partials, p.n_blocks, a.sqnorm, st);
}

hipError_t launch_sqnorm_bf16(const ApplyArgs &a, void *ws, hipStream_t st) {
    switch (a.R) {
    case 32: return sqnorm_r<32>(a, ws, st);
    case 64: return sqnorm_r<64>(a, ws, st);
    case 128: return sqnorm_r<128>(a, ws, st);
    case 256: return sqnorm_r<256>(a, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
