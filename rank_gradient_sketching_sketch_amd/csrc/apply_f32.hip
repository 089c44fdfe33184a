// fp32 twin of the apply passes: Ghat = S A rebuilt in fp32 (no
// reduced-precision products), then pass 1 (rowsq, controller partials) or
// pass 2 (RowAdam update from v'). Same definitions as the bf16 kernels ("NVIDIA's
// LoGRA fits RL post-training...", sections "What happened" and "Why it
// matters"; "LoGRA: Scaling LLM Reinforcement Learning...", paragraph "Step
// control."). A workgroup owns 8 rows; each of its 256 threads takes one
// (row, column) pair per 32-column step and sums over the rank in order.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

constexpr int kF32Rows = 8;
constexpr int kF32MaxR = 1024;

template <int MODE, bool WBF16>
__global__ __launch_bounds__(256) void apply_f32_kernel(ApplyArgs a) {
    __shared__ float srows[kF32Rows][kF32MaxR];
    __shared__ uint64_t wl[kF32MaxR];
    __shared__ float coef_s[kF32Rows];
    __shared__ float term_s[kF32Rows];
    const int tid = threadIdx.x;
    const int q = tid >> 5, jj = tid & 31;
    const int R = a.R;
    const int D = static_cast<int>(a.D), K = static_cast<int>(a.K);
    const int i0 = blockIdx.x * kF32Rows;
    const int i = i0 + q;
    for (int idx = tid; idx < kF32Rows * R; idx += 256) {
        const int rr = idx / R, l = idx - rr * R;
        const int ii = i0 + rr;
        srows[rr][l] = ii < D ? a.S[static_cast<int64_t>(ii) * R + l] : 0.f;
    }
    if (MODE == 1 && tid < kF32Rows) {
        const int ii = i0 + tid;
        float coef = 0.f;
        if (ii < D) {
            const float u = 1.f / (sqrtf(a.v_new_in[ii]) + a.eps);
            coef = a.lr_scale * a.c * u;
        }
        coef_s[tid] = coef;
    }
    float ss = 0.f;
    for (int j0 = 0; j0 < K; j0 += 32) {
        if ((j0 & 63) == 0) {
            __syncthreads();
            for (int l = tid; l < R; l += 256)
                wl[l] = sign_word(a.key, static_cast<uint32_t>(l), static_cast<uint32_t>(j0 >> 6));
            __syncthreads();
        }
        const int j = j0 + jj;
        const int bit = j & 63;
        float gsum = 0.f;
        for (int l = 0; l < R; ++l) {
            const float sg = ((wl[l] >> bit) & 1ull) ? -1.f : 1.f;
            gsum = fmaf(sg, srows[q][l], gsum);
        }
        if (i < D && j < K) {
            if (MODE == 0) {
                ss = fmaf(gsum, gsum, ss);
            } else {
                const float cf = coef_s[q];
                const int64_t off = static_cast<int64_t>(i) * a.ldw + j;
                if (WBF16) {
                    uint16_t *wp = static_cast<uint16_t *>(a.W) + off;
                    const float w = __uint_as_float(static_cast<uint32_t>(*wp) << 16);
                    *wp = __builtin_bit_cast(uint16_t, (__bf16)fmaf(-cf, gsum, w));
                } else {
                    float *wp = static_cast<float *>(a.W) + off;
                    *wp = fmaf(-cf, gsum, *wp);
                }
            }
        }
    }
    if (MODE == 0) {
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off, 64);
        if (jj == 0) {
            float term = 0.f;
            if (i < D) {
                const float rq = (a.c * a.c) * ss;
                if (a.rowsq_out) a.rowsq_out[i] = rq;
                const float vn = a.beta2 * a.v_in[i] + (1.f - a.beta2) * (rq / static_cast<float>(K));
                a.v_new_out[i] = vn;
                const float u = 1.f / (sqrtf(vn) + a.eps);
                term = rq * u * u;
            }
            term_s[q] = term;
        }
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
            for (int r = 0; r < kF32Rows; ++r) t += term_s[r];
            a.partials[blockIdx.x] = t;
        }
    }
}

int apply_blocks_f32(int64_t D) { return static_cast<int>((D + kF32Rows - 1) / kF32Rows); }

hipError_t launch_apply_f32(int mode, const ApplyArgs &a, hipStream_t st) {
    if (a.R > kF32MaxR) return hipErrorInvalidValue;
    const dim3 grid(apply_blocks_f32(a.D)), block(256);
    if (mode == 0)
        hipLaunchKernelGGL((apply_f32_kernel<0, false>), grid, block, 0, st, a);
    else if (a.w_bf16)
        hipLaunchKernelGGL((apply_f32_kernel<1, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((apply_f32_kernel<1, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace logra
