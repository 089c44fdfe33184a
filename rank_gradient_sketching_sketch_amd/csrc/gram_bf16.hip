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

// M_off[l][m] (bf16, row-major r x r, zero diagonal). A workgroup owns a 16 x
// 16 tile of (l, m); the sign words of its 32 rows are hashed into LDS 64
// columns-blocks at a time and each thread counts the sign differences of
// its pair.
constexpr int kGramChunk = 64;   // 64-bit words per row per chunk

__global__ __launch_bounds__(256) void gram_kernel(uint64_t key, int R, int K, uint16_t *__restrict__ M) {
    __shared__ uint64_t wl[16][kGramChunk];
    __shared__ uint64_t wm[16][kGramChunk];
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
                w = sign_word(key, static_cast<uint32_t>((which ? m0 : l0) + row),
                              static_cast<uint32_t>(b0 + bb));
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

// One wave per 32 rows of S (two 16-row blocks), four waves per workgroup.
// Y (32 x r) = S_bf16 M_off accumulates on the matrix cores one 16-column
// block at a time; each lane dots its Y entries with the fp32 S entries at the
// same place and also sums their squares, then the 16 lanes of a row add up.
template <int R>
__global__ __launch_bounds__(256) void rowsq_gram_kernel(const float *__restrict__ S, int D, int K,
                                                         const uint16_t *__restrict__ M, float c,
                                                         const float *__restrict__ v, float beta2,
                                                         float eps, float *__restrict__ rowsq,
                                                         float *__restrict__ partials) {
    constexpr int KS = R / 32;   // 32-wide steps of the rank
    constexpr int NB = R / 16;   // 16-wide column blocks of Y
    __shared__ float terms[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int i0 = blockIdx.x * 128 + wave * 32;

    // A fragments: lane (n, g) of block mb, step s = S[i0 + 16 mb + n][32 s + 8 g .. +7] in bf16
    u32x4_t af[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int i = i0 + 16 * mb + n;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (i < D) {
                const float *p = S + static_cast<int64_t>(i) * R + 32 * s + 8 * g;
                const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p);
                const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(p + 4);
                af[mb][s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                                    pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
            } else {
                af[mb][s] = zero_u32x4();
            }
        }
    }
    // row of Y held by lane (n, g), block mb, element e: i0 + 16 mb + 4 g + e
    float ydot[2][4], ssq[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) ydot[mb][e] = ssq[mb][e] = 0.f;

    // B fragments: M_off[32 s + 8 g + e][16 nb + n] = M_off[16 nb + n][32 s + 8 g + e]
    // (M is symmetric); fetched one column block ahead, with the fp32 S entries
    auto fetch = [&](int nb, u32x4_t (&bf)[KS], float (&sv)[2][4]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            bf[s] = load_u32x4(M + static_cast<size_t>(16 * nb + n) * R + 32 * s + 8 * g);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = min(i0 + 16 * mb + 4 * g + e, D - 1);   // rows past d are dropped below
                sv[mb][e] = S[static_cast<int64_t>(i) * R + 16 * nb + n];
            }
    };
    u32x4_t bf[KS], bf_n[KS];
    float sv[2][4], sv_n[2][4];
    fetch(0, bf, sv);
#pragma unroll 1
    for (int nb = 0; nb < NB; ++nb) {
        if (nb + 1 < NB) fetch(nb + 1, bf_n, sv_n);
        f32x4_t acc[2] = {zero_f32x4(), zero_f32x4()};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) acc[mb] = mfma_bf16(af[mb][s], bf[s], acc[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ydot[mb][e] = fmaf(sv[mb][e], acc[mb][e], ydot[mb][e]);
                ssq[mb][e] = fmaf(sv[mb][e], sv[mb][e], ssq[mb][e]);
            }
#pragma unroll
        for (int s = 0; s < KS; ++s) bf[s] = bf_n[s];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[mb][e] = sv_n[mb][e];
    }
    // add the 16 lanes of each row (lanes g*16 .. g*16+15), fixed butterfly order
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                ydot[mb][e] += __shfl_xor(ydot[mb][e], off, 64);
                ssq[mb][e] += __shfl_xor(ssq[mb][e], off, 64);
            }
    // lane n == e writes row 16 mb + 4 g + e
    float term = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + 16 * mb + 4 * g + e;
            if (n == e && i < D) {
                const float rq = (c * c) * fmaf(static_cast<float>(K), ssq[mb][e], ydot[mb][e]);
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
    const size_t align = 256;
    p.partial_bytes = (static_cast<size_t>(p.n_blocks) * 4 + align - 1) / align * align;
    p.gram_bytes = static_cast<size_t>(R) * R * 2;
    (void)K;
    return p;
}

template <int R>
static hipError_t sqnorm_r(const ApplyArgs &a, void *ws, hipStream_t st) {
    const SqnormPlan p = plan_sqnorm_bf16(a.D, a.K, R);
    char *base = static_cast<char *>(ws);
    float *partials = reinterpret_cast<float *>(base);
    uint16_t *M = reinterpret_cast<uint16_t *>(base + p.partial_bytes);
    hipLaunchKernelGGL(gram_kernel, dim3(R / 16, R / 16), dim3(256), 0, st, a.key, R,
                       static_cast<int>(a.K), M);
    hipLaunchKernelGGL(rowsq_gram_kernel<R>, dim3(p.n_blocks), dim3(256), 0, st, a.S,
                       static_cast<int>(a.D), static_cast<int>(a.K), M, a.c, a.v_in, a.beta2, a.eps,
                       a.rowsq_out, partials);
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
