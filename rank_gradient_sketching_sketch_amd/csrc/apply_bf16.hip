// Apply pass 2 for bf16 compute: rebuild Ghat = S A tile by tile on the
// matrix cores and apply RowAdam, W_ij -= lr * scale * Ghat_ij / (sqrt(v'_i) + eps).
//
// The update estimate S A exists only while it is applied ("NVIDIA's LoGRA
// fits RL post-training of a 27B model onto a single eight-GPU node", section
// "Why it matters"); RowAdam keeps one running second moment per row and no
// first moment (same page, "What happened" and "Why it matters").
//
// Layout: a workgroup (4 waves) owns 64 rows of W and a range of 128-column
// tiles; the grid is (row tiles) x (column ranges) so that every CU gets
// several workgroups. The MFMA computes Ghat^T tiles: A operand = sign
// fragments (16 columns j x 32 rank indices l), B operand = S^T (32 l x 16
// rows i; S rounded to bf16 once per workgroup and kept in registers), so each
// lane's accumulator holds consecutive columns of one row of W and W moves in
// 16-byte vectors. MFMA row m of column block mb stands for column
// 8*(m/4) + 4*mb + m%4 of the wave's 32, which puts columns 8g .. 8g+7 of row
// i in lane (i, g). The sign words of the current 128 columns (2 x r words)
// are hashed into LDS once per workgroup and tile. W goes through a buffer
// view (rows past d and columns past k read as zero and are not written), and
// the next tile's W is requested before the current tile's products, so the
// W stream overlaps the matrix work instead of waiting on it.
//
// Every workgroup of a row tile reads v and rowsq to form u_i; v itself is
// committed by a separate small pass once all of them are done.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

constexpr uint32_t kOobOff = 0x80000000u;

template <int R, bool WBF16>
__global__ __launch_bounds__(256) void rowadam_bf16_kernel(ApplyArgs a, int it_per) {
    constexpr int KS = R / 32;                 // 32-wide steps of the rank
    constexpr int WV = WBF16 ? 1 : 2;          // 16-byte vectors per 8 columns of W
    __shared__ uint32_t words[2][2][2][R];     // [buffer][column block][half][l]
    __shared__ float coef_s[64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int D = static_cast<int>(a.D), K = static_cast<int>(a.K);
    const int i_base = blockIdx.x * 64;
    const int niter = (K + 127) / 128;
    const int it_begin = blockIdx.y * it_per;
    const int it_end = min(niter, it_begin + it_per);

    // S^T fragments: lane (n, g) of block nb, step s holds S[i][32s + 8g .. +7], i = i_base+16nb+n
    u32x4_t sf[4][KS];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int i = min(i_base + 16 * nb + n, D - 1);   // rows past d compute junk, never stored
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const float *p = a.S + static_cast<int64_t>(i) * R + 32 * s + 8 * g;
            const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p);
            const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(p + 4);
            sf[nb][s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                                pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
        }
    }
    if (tid < 64) {
        const int i = i_base + tid;
        float coef = 0.f;
        if (i < D) {
            const float vn = a.beta2 * a.v[i] + (1.f - a.beta2) * (a.rowsq_in[i] / static_cast<float>(K));
            coef = a.lr_scale * a.c / (sqrtf(vn) + a.eps);
        }
        coef_s[tid] = coef;
    }

    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.W, 0, static_cast<int>(static_cast<int64_t>(D) * a.ldw * (WBF16 ? 2 : 4)), 0x00020000);
    // byte offset of this lane's 8 columns in row block nb, tile it (kOobOff if masked)
    auto w_off = [&](int it, int nb) -> uint32_t {
        const int i = i_base + 16 * nb + n;
        const int jc = it * 128 + 32 * wave + 8 * g;
        const bool ok = it < it_end && i < D && jc < K;
        return ok ? static_cast<uint32_t>((static_cast<int64_t>(i) * a.ldw + jc) * (WBF16 ? 2 : 4))
                  : kOobOff;
    };
    auto w_load = [&](int it, u32x4_t (&w)[4][WV]) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const uint32_t off = w_off(it, nb);
#pragma unroll
            for (int h = 0; h < WV; ++h)
                w[nb][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                           w_rs, off == kOobOff ? off : off + 16 * h, 0, 0));
        }
    };

    // bit of column (j0 + 32*wave + jmap(mb, n)) inside the wave's 32-bit half word
    const int jbit = 8 * (n >> 2) + (n & 3);
    const int b2 = wave >> 1, half = wave & 1;

    u32x4_t wcur[4][WV], wnxt[4][WV];
    w_load(it_begin, wcur);
    for (int it = it_begin; it < it_end; ++it) {
        const int j0 = it * 128;
        const int buf = it & 1;
        for (int idx = tid; idx < 2 * R; idx += 256) {
            const int bb = idx / R, l = idx - bb * R;
            const uint64_t w = sign_word(a.key, static_cast<uint32_t>(l),
                                         static_cast<uint32_t>((j0 >> 6) + bb));
            words[buf][bb][0][l] = static_cast<uint32_t>(w);
            words[buf][bb][1][l] = static_cast<uint32_t>(w >> 32);
        }
        w_load(it + 1, wnxt);   // next tile's W in flight during this tile's products
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
        // lane (n, g) of block nb holds Ghat/c for row i_base+16nb+n, columns
        // jc .. jc+7 (acc[0] the first four, acc[1] the next four)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const float cf = coef_s[16 * nb + n];
            const f32x4_t x0 = acc[0][nb], x1 = acc[1][nb];
            const uint32_t off = w_off(it, nb);
            if (WBF16) {
                const u32x4_t wv = wcur[nb][0];
                u32x4_t o;
                o.x = pack_bf16x2(fmaf(-cf, x0.x, bf16_lo(wv.x)), fmaf(-cf, x0.y, bf16_hi(wv.x)));
                o.y = pack_bf16x2(fmaf(-cf, x0.z, bf16_lo(wv.y)), fmaf(-cf, x0.w, bf16_hi(wv.y)));
                o.z = pack_bf16x2(fmaf(-cf, x1.x, bf16_lo(wv.z)), fmaf(-cf, x1.y, bf16_hi(wv.z)));
                o.w = pack_bf16x2(fmaf(-cf, x1.z, bf16_lo(wv.w)), fmaf(-cf, x1.w, bf16_hi(wv.w)));
                __builtin_amdgcn_raw_buffer_store_b128(o, w_rs, off, 0, 0);
            } else {
                f32x4_t w0v = __builtin_bit_cast(f32x4_t, wcur[nb][0]);
                f32x4_t w1v = __builtin_bit_cast(f32x4_t, wcur[nb][WV - 1]);
                w0v.x = fmaf(-cf, x0.x, w0v.x); w0v.y = fmaf(-cf, x0.y, w0v.y);
                w0v.z = fmaf(-cf, x0.z, w0v.z); w0v.w = fmaf(-cf, x0.w, w0v.w);
                w1v.x = fmaf(-cf, x1.x, w1v.x); w1v.y = fmaf(-cf, x1.y, w1v.y);
                w1v.z = fmaf(-cf, x1.z, w1v.z); w1v.w = fmaf(-cf, x1.w, w1v.w);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w0v), w_rs, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w1v), w_rs,
                                                      off == kOobOff ? off : off + 16, 0, 0);
            }
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int h = 0; h < WV; ++h) wcur[nb][h] = wnxt[nb][h];
    }
}

// v <- beta2 v + (1 - beta2) rowsq / k, after every workgroup of the apply has read v.
__global__ __launch_bounds__(256) void commit_v_kernel(float *__restrict__ v, const float *__restrict__ rowsq,
                                                       int D, float beta2, float inv_k) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < D) v[i] = beta2 * v[i] + (1.f - beta2) * (rowsq[i] * inv_k);
}

hipError_t launch_commit_v(float *v, const float *rowsq, int64_t D, int64_t K, float beta2, hipStream_t st) {
    hipLaunchKernelGGL(commit_v_kernel, dim3((D + 255) / 256), dim3(256), 0, st, v, rowsq,
                       static_cast<int>(D), beta2, 1.f / static_cast<float>(K));
    return hipGetLastError();
}

template <int R>
static hipError_t rowadam_r(const ApplyArgs &a, hipStream_t st) {
    const int row_tiles = static_cast<int>((a.D + 63) / 64);
    const int niter = static_cast<int>((a.K + 127) / 128);
    // about four workgroups per compute unit in total
    int n_ranges = (1024 + row_tiles - 1) / row_tiles;
    if (n_ranges > niter) n_ranges = niter;
    if (n_ranges < 1) n_ranges = 1;
    const int it_per = (niter + n_ranges - 1) / n_ranges;
    n_ranges = (niter + it_per - 1) / it_per;
    const dim3 grid(row_tiles, n_ranges), block(256);
    if (a.w_bf16)
        hipLaunchKernelGGL((rowadam_bf16_kernel<R, true>), grid, block, 0, st, a, it_per);
    else
        hipLaunchKernelGGL((rowadam_bf16_kernel<R, false>), grid, block, 0, st, a, it_per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_commit_v(a.v, a.rowsq_in, a.D, a.K, a.beta2, st);
}

hipError_t launch_rowadam_bf16(const ApplyArgs &a, hipStream_t st) {
    switch (a.R) {
    case 32: return rowadam_r<32>(a, st);
    case 64: return rowadam_r<64>(a, st);
    case 128: return rowadam_r<128>(a, st);
    case 256: return rowadam_r<256>(a, st);
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
