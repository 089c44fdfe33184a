// Rebuild Ghat = S A tile by tile on the matrix cores and either reduce it
// (pass 1) or apply RowAdam with it (pass 2).
//
// The update estimate S A exists only while the update is applied ("NVIDIA's
// LoGRA fits RL post-training of a 27B model onto a single eight-GPU node",
// section "Why it matters"); RowAdam keeps one running second moment per row
// and no first moment (same page, "What happened" and "Why it matters"). The
// step controller reads sum_ij (Ghat_ij / (sqrt(v'_i) + eps))^2 before the
// update ("LoGRA: Scaling LLM Reinforcement Learning...", paragraph "Step
// control.").
//
// Layout of one workgroup (4 waves): 64 rows of W and a sweep over all k in
// 128-column steps, 32 columns per wave. The MFMA computes Ghat^T tiles:
// A operand = sign fragments (16 columns j x 32 rank indices l), B operand =
// S^T (32 l x 16 rows i, S rounded to bf16 once and kept in registers for the
// whole sweep), so each lane's accumulator holds consecutive columns of one
// row of W and the W traffic is 16-byte vectors. MFMA row m of column block
// mb stands for column 8*(m/4) + 4*mb + m%4 of the wave's 32, which puts
// columns 8g .. 8g+7 of row i in lane (i, g). The sign words of the current
// 128 columns (2 x r words) are hashed once per workgroup into LDS.
//
// Pass 1 writes rowsq_i = sum_j Ghat_ij^2 and one partial of the controller's
// reduction per workgroup; pass 2 commits v' and writes W.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

template <int R, int MODE, bool WBF16>
__global__ __launch_bounds__(256) void apply_bf16_kernel(ApplyArgs a) {
    constexpr int KS = R / 32;   // 32-wide steps of the rank dimension
    __shared__ uint32_t words[2][2][2][R];   // [buffer][column block][half][l]
    __shared__ float coef_s[64];
    __shared__ float red[4][64];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int D = static_cast<int>(a.D), K = static_cast<int>(a.K);
    const int i_base = blockIdx.x * 64;

    // S^T fragments: lane (n, g) of block nb, step s holds S[i][32s + 8g .. +7], i = i_base+16nb+n
    u32x4_t sf[4][KS];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int i = i_base + 16 * nb + n;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (i < D) {
                const float *p = a.S + static_cast<int64_t>(i) * R + 32 * s + 8 * g;
                const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p);
                const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(p + 4);
                sf[nb][s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                                    pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
            } else {
                sf[nb][s] = zero_u32x4();
            }
        }
    }

    if (MODE == 1 && tid < 64) {
        const int i = i_base + tid;
        float coef = 0.f;
        if (i < D) {
            const float vn = a.beta2 * a.v[i] + (1.f - a.beta2) * (a.rowsq_in[i] / static_cast<float>(K));
            const float u = 1.f / (sqrtf(vn) + a.eps);
            coef = a.lr_scale * a.c * u;
            a.v[i] = vn;
        }
        coef_s[tid] = coef;
    }

    // bit of column (j0 + 32*wave + jmap(mb, n)) inside the wave's 32-bit half word
    const int jbit = 8 * (n >> 2) + (n & 3);
    const int b2 = wave >> 1, half = wave & 1;
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    const int niter = (K + 127) / 128;

    for (int it = 0; it < niter; ++it) {
        const int j0 = it * 128;
        const int buf = it & 1;
        for (int idx = tid; idx < 2 * R; idx += 256) {
            const int bb = idx / R, l = idx - bb * R;
            const uint64_t w = sign_word(a.key, static_cast<uint32_t>(l),
                                         static_cast<uint32_t>((j0 >> 6) + bb));
            words[buf][bb][0][l] = static_cast<uint32_t>(w);
            words[buf][bb][1][l] = static_cast<uint32_t>(w >> 32);
        }
        __syncthreads();
        const uint32_t *wp = &words[buf][b2][half][0];
        f32x4_t acc[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = zero_f32x4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // words of rank rows l = 32s + 8g .. +7 (same for all 16 lanes of a group)
            const u32x4_t w0 = *reinterpret_cast<const u32x4_t *>(wp + 32 * s + 8 * g);
            const u32x4_t w1 = *reinterpret_cast<const u32x4_t *>(wp + 32 * s + 8 * g + 4);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int sh = jbit + 4 * mb;
                u32x4_t af;
                af.x = 0x3F803F80u | (((w0.x >> sh) & 1u) << 15) | (((w0.y >> sh) & 1u) << 31);
                af.y = 0x3F803F80u | (((w0.z >> sh) & 1u) << 15) | (((w0.w >> sh) & 1u) << 31);
                af.z = 0x3F803F80u | (((w1.x >> sh) & 1u) << 15) | (((w1.y >> sh) & 1u) << 31);
                af.w = 0x3F803F80u | (((w1.z >> sh) & 1u) << 15) | (((w1.w >> sh) & 1u) << 31);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(af, sf[nb][s], acc[mb][nb]);
            }
        }
        // lane (n, g) of block nb now holds Ghat/c for row i_base+16nb+n,
        // columns jc .. jc+7 (acc[0] the first four, acc[1] the next four)
        const int jc = j0 + 32 * wave + 8 * g;
        if (jc < K) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int i = i_base + 16 * nb + n;
                if (i >= D) continue;
                const f32x4_t x0 = acc[0][nb], x1 = acc[1][nb];
                if (MODE == 0) {
                    float t = ss[nb];
                    t = fmaf(x0.x, x0.x, t); t = fmaf(x0.y, x0.y, t);
                    t = fmaf(x0.z, x0.z, t); t = fmaf(x0.w, x0.w, t);
                    t = fmaf(x1.x, x1.x, t); t = fmaf(x1.y, x1.y, t);
                    t = fmaf(x1.z, x1.z, t); t = fmaf(x1.w, x1.w, t);
                    ss[nb] = t;
                } else {
                    const float cf = coef_s[16 * nb + n];
                    if (WBF16) {
                        uint16_t *wr = static_cast<uint16_t *>(a.W) + static_cast<int64_t>(i) * a.ldw + jc;
                        const u32x4_t wv = *reinterpret_cast<const u32x4_t *>(wr);
                        u32x4_t o;
                        o.x = pack_bf16x2(fmaf(-cf, x0.x, bf16_lo(wv.x)), fmaf(-cf, x0.y, bf16_hi(wv.x)));
                        o.y = pack_bf16x2(fmaf(-cf, x0.z, bf16_lo(wv.y)), fmaf(-cf, x0.w, bf16_hi(wv.y)));
                        o.z = pack_bf16x2(fmaf(-cf, x1.x, bf16_lo(wv.z)), fmaf(-cf, x1.y, bf16_hi(wv.z)));
                        o.w = pack_bf16x2(fmaf(-cf, x1.z, bf16_lo(wv.w)), fmaf(-cf, x1.w, bf16_hi(wv.w)));
                        *reinterpret_cast<u32x4_t *>(wr) = o;
                    } else {
                        float *wr = static_cast<float *>(a.W) + static_cast<int64_t>(i) * a.ldw + jc;
                        f32x4_t w0v = *reinterpret_cast<const f32x4_t *>(wr);
                        f32x4_t w1v = *reinterpret_cast<const f32x4_t *>(wr + 4);
                        w0v.x = fmaf(-cf, x0.x, w0v.x); w0v.y = fmaf(-cf, x0.y, w0v.y);
                        w0v.z = fmaf(-cf, x0.z, w0v.z); w0v.w = fmaf(-cf, x0.w, w0v.w);
                        w1v.x = fmaf(-cf, x1.x, w1v.x); w1v.y = fmaf(-cf, x1.y, w1v.y);
                        w1v.z = fmaf(-cf, x1.z, w1v.z); w1v.w = fmaf(-cf, x1.w, w1v.w);
                        *reinterpret_cast<f32x4_t *>(wr) = w0v;
                        *reinterpret_cast<f32x4_t *>(wr + 4) = w1v;
                    }
                }
            }
        }
    }

    if (MODE == 0) {
        // rows: lanes (n, g) -> add the four g groups, then the four waves, in fixed order
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            float t = ss[nb];
            t += __shfl_xor(t, 16, 64);
            t += __shfl_xor(t, 32, 64);
            if (g == 0) red[wave][16 * nb + n] = t;
        }
        __syncthreads();
        if (tid < 64) {
            const int i = i_base + tid;
            float term = 0.f;
            if (i < D) {
                const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
                const float rq = (a.c * a.c) * tot;
                a.rowsq_out[i] = rq;
                const float vn = a.beta2 * a.v_in[i] + (1.f - a.beta2) * (rq / static_cast<float>(K));
                const float u = 1.f / (sqrtf(vn) + a.eps);
                term = rq * u * u;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) term += __shfl_xor(term, off, 64);
            if (tid == 0) a.partials[blockIdx.x] = term;
        }
    }
}

int apply_blocks_bf16(int64_t D) { return static_cast<int>((D + 63) / 64); }

template <int R>
static hipError_t apply_bf16_r(int mode, const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(apply_blocks_bf16(a.D)), block(256);
    if (mode == 0) {
        hipLaunchKernelGGL((apply_bf16_kernel<R, 0, false>), grid, block, 0, st, a);
    } else if (a.w_bf16) {
        hipLaunchKernelGGL((apply_bf16_kernel<R, 1, true>), grid, block, 0, st, a);
    } else {
        hipLaunchKernelGGL((apply_bf16_kernel<R, 1, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_apply_bf16(int mode, const ApplyArgs &a, hipStream_t st) {
    switch (a.R) {
    case 32: return apply_bf16_r<32>(mode, a, st);
    case 64: return apply_bf16_r<64>(mode, a, st);
    case 128: return apply_bf16_r<128>(mode, a, st);
    case 256: return apply_bf16_r<256>(mode, a, st);
    default: return hipErrorInvalidValue;
    }
}

// sqnorm = sum of the per-workgroup partials, in a fixed order.
__global__ __launch_bounds__(256) void sqnorm_final_kernel(const float *__restrict__ part, int n,
                                                           float *__restrict__ out) {
    __shared__ float red[256];
    float t = 0.f;
    for (int i = threadIdx.x; i < n; i += 256) t += part[i];
    red[threadIdx.x] = t;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

hipError_t launch_sqnorm_final(const float *partials, int n, float *out, hipStream_t st) {
    hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(256), 0, st, partials, n, out);
    return hipGetLastError();
}

}  // namespace logra
