// Sketch accumulation S (+)= dY^T (X A^T), bf16 inputs, on the matrix cores.
//
// The sketch of a weight gradient G = dY^T X is S = G A^T, summed as
// microbatches arrive, so G itself is never formed ("NVIDIA's LoGRA fits RL
// post-training of a 27B model onto a single eight-GPU node", section "Why it
// matters"; "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", paragraph "Gradient sketches."). Two products, both dense
// contractions on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation:
//
//   stage 1   P = c * X Sigma^T  (T x r, contraction over k). A's sign tiles
//             are made in registers from the counter hash: one 64-bit word per
//             lane per 64 columns, shuffled to the lanes of each 16-column
//             block, bytes expanded to bf16 +-1. The k range is split across
//             workgroups so that a microbatch fills the GPU; partial sums go to
//             the workspace and a finalize pass adds them in a fixed order,
//             scales by c and rounds P to bf16 (nearest even) in a layout whose
//             16-byte chunks are exactly the stage-2 operand fragments.
//   stage 2   S (+)= dY^T P  (d x r, contraction over the tokens): the fold
//             kernel in fold_bf16.hip.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

template <int R>
struct SketchShape {
    static constexpr int NB = R / 16;            // 16-wide column blocks of r
    static constexpr int WN = NB < 4 ? NB : 4;   // waves across r
    static constexpr int NBW = NB / WN;          // column blocks per wave
    static constexpr int WM = 4 / WN;            // waves across rows
    static_assert(R % 32 == 0 && R <= 256, "bf16 sketch supports r in {32,64,128,256}");
};

constexpr int kS1RowBlocks = 8;   // 16-row MFMA blocks per wave in stage 1 (128 tokens)

// ---------------------------------------------------------------- stage 1 --
template <int R>
__global__ __launch_bounds__(256) void stage1_bf16_kernel(
    const uint16_t *__restrict__ X, int64_t ldx, int T, int K, uint64_t key, int kchunk,
    float *__restrict__ part, int t_pad) {
    using Sh = SketchShape<R>;
    constexpr int MBW = kS1RowBlocks;
    constexpr int NBW = Sh::NBW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / Sh::WN, wn = wave % Sh::WN;
    const int n = lane & 15, g = lane >> 4;
    const int t_base = blockIdx.x * (Sh::WM * 128) + wm * 128;
    const int l_base = wn * NBW * 16;
    const int split = blockIdx.y;
    const int j_begin = split * kchunk;
    const int j_end = min(K, j_begin + kchunk);

    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = zero_f32x4();

    const uint16_t *xrow[MBW];
    bool rowok[MBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int t = t_base + 16 * mb + n;
        rowok[mb] = t < T;
        xrow[mb] = X + static_cast<int64_t>(rowok[mb] ? t : 0) * ldx;
    }

    const int s_begin = j_begin >> 5;           // 32-column steps; j_begin % 64 == 0
    const int s_end = (j_end + 31) >> 5;

    u32x4_t a_cur[MBW];
    {
        const int jj = (s_begin << 5) + 8 * g;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            a_cur[mb] = (rowok[mb] && jj < j_end) ? load_u32x4(xrow[mb] + jj) : zero_u32x4();
    }
    uint32_t wlo[NBW], whi[NBW];
    const uint32_t my_l = static_cast<uint32_t>(l_base + (lane % (NBW * 16)));

    for (int s = s_begin; s < s_end; ++s) {
        u32x4_t a_nxt[MBW];
        if (s + 1 < s_end) {
            const int jj = ((s + 1) << 5) + 8 * g;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                a_nxt[mb] = (rowok[mb] && jj < j_end) ? load_u32x4(xrow[mb] + jj) : zero_u32x4();
        }
        if (((s - s_begin) & 1) == 0) {
            // one sign word per lane: row my_l, columns 64*(s/2) .. +63
            const uint64_t w = sign_word(key, my_l, static_cast<uint32_t>(s >> 1));
            const int lo = static_cast<int>(static_cast<uint32_t>(w));
            const int hi = static_cast<int>(static_cast<uint32_t>(w >> 32));
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int src = nb * 16 + n;
                wlo[nb] = static_cast<uint32_t>(__shfl(lo, src, 64));
                whi[nb] = static_cast<uint32_t>(__shfl(hi, src, 64));
            }
        }
        u32x4_t bfrag[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const uint32_t dw = (s & 1) ? whi[nb] : wlo[nb];
            bfrag[nb] = signs8_to_bf16((dw >> (8 * g)) & 0xFFu);
        }
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = mfma_bf16(a_cur[mb], bfrag[nb], acc[mb][nb]);
        if (s + 1 < s_end) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) a_cur[mb] = a_nxt[mb];
        }
    }

    // partial tile -> part[split][t/32][l][t%32] (fp32, 4 consecutive tokens per lane)
    const size_t tb_count = static_cast<size_t>(t_pad >> 5);
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int t = t_base + 16 * mb + 4 * g;
        const size_t tb = static_cast<size_t>(t >> 5);
        const int tt = t & 31;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int l = l_base + 16 * nb + n;
            float *dst = part + ((static_cast<size_t>(split) * tb_count + tb) * R + l) * 32 + tt;
            *reinterpret_cast<f32x4_t *>(dst) = acc[mb][nb];
        }
    }
}

// P[t/32][l][t%32] = bf16(c * sum over splits of the partials), splits added in order.
template <int R>
__global__ __launch_bounds__(256) void stage1_finalize_kernel(const float *__restrict__ part, int ks,
                                                              int t_pad, float c,
                                                              uint16_t *__restrict__ P) {
    const size_t total = static_cast<size_t>(t_pad >> 5) * R * 4;   // 8 tokens per thread
    const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const size_t base = idx * 8;
    const size_t slab = static_cast<size_t>(t_pad) * R;
    f32x4_t s0 = zero_f32x4(), s1 = zero_f32x4();
    for (int sp = 0; sp < ks; ++sp) {
        const float *p = part + sp * slab + base;
        s0 += *reinterpret_cast<const f32x4_t *>(p);
        s1 += *reinterpret_cast<const f32x4_t *>(p + 4);
    }
    u32x4_t o;
    o.x = pack_bf16x2(c * s0.x, c * s0.y);
    o.y = pack_bf16x2(c * s0.z, c * s0.w);
    o.z = pack_bf16x2(c * s1.x, c * s1.y);
    o.w = pack_bf16x2(c * s1.z, c * s1.w);
    *reinterpret_cast<u32x4_t *>(P + base) = o;
}

// ----------------------------------------------------------------- plans --
static int stage1_tile_m(int R) {
    const int nb = R / 16;
    const int wn = nb < 4 ? nb : 4;
    return (4 / wn) * 128;
}

Stage1Plan plan_stage1_bf16(int64_t T, int64_t K, int R) {
    Stage1Plan p;
    if (T <= 0) return p;
    p.tile_m = stage1_tile_m(R);
    p.n_mtiles = static_cast<int>((T + p.tile_m - 1) / p.tile_m);
    const int nkb = static_cast<int>((K + 63) / 64);
    const int target = 512;   // about two workgroups per compute unit
    int ks = (target + p.n_mtiles - 1) / p.n_mtiles;
    if (ks < 1) ks = 1;
    if (ks > nkb) ks = nkb;
    const int blocks_per = (nkb + ks - 1) / ks;
    p.ks = (nkb + blocks_per - 1) / blocks_per;
    p.kchunk = blocks_per * 64;
    p.t_pad = static_cast<int64_t>(p.n_mtiles) * p.tile_m;
    p.part_bytes = static_cast<size_t>(p.ks) * p.t_pad * R * 4;
    p.p_bytes = static_cast<size_t>(p.t_pad) * R * 2;
    return p;
}

template <int R>
static hipError_t project_bf16_r(int64_t T, int64_t K, uint64_t key, float c, const uint16_t *X,
                                 int64_t ldx, void *ws, hipStream_t st) {
    const Stage1Plan p = plan_stage1_bf16(T, K, R);
    float *part = static_cast<float *>(ws);
    uint16_t *P = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + p.part_bytes);
    hipLaunchKernelGGL(stage1_bf16_kernel<R>, dim3(p.n_mtiles, p.ks), dim3(256), 0, st, X, ldx,
                       static_cast<int>(T), static_cast<int>(K), key, p.kchunk, part,
                       static_cast<int>(p.t_pad));
    const size_t fin_threads = static_cast<size_t>(p.t_pad / 32) * R * 4;
    hipLaunchKernelGGL(stage1_finalize_kernel<R>, dim3((fin_threads + 255) / 256), dim3(256), 0, st,
                       part, p.ks, static_cast<int>(p.t_pad), c, P);
    return hipGetLastError();
}

template <int R>
static hipError_t fold_bf16_r(int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                              float *S, int accumulate, const void *ws, hipStream_t st) {
    const Stage1Plan p = plan_stage1_bf16(T, K, R);
    const char *base = static_cast<const char *>(ws);
    const uint16_t *P = reinterpret_cast<const uint16_t *>(base + p.part_bytes);
    float *part = reinterpret_cast<float *>(const_cast<char *>(base) + p.part_bytes + p.p_bytes);
    return launch_fold_bf16_tiles(R, T, D, dY, lddy, P, static_cast<int>(p.t_pad / 32), S, accumulate,
                                  part, st);
}

hipError_t launch_project_bf16(int R, int64_t T, int64_t K, uint64_t key, float c, const uint16_t *X,
                               int64_t ldx, void *ws, hipStream_t st) {
    switch (R) {
    case 32: return project_bf16_r<32>(T, K, key, c, X, ldx, ws, st);
    case 64: return project_bf16_r<64>(T, K, key, c, X, ldx, ws, st);
    case 128: return project_bf16_r<128>(T, K, key, c, X, ldx, ws, st);
    case 256: return project_bf16_r<256>(T, K, key, c, X, ldx, ws, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fold_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                            float *S, int accumulate, const void *ws, hipStream_t st) {
    switch (R) {
    case 32: return fold_bf16_r<32>(T, D, K, dY, lddy, S, accumulate, ws, st);
    case 64: return fold_bf16_r<64>(T, D, K, dY, lddy, S, accumulate, ws, st);
    case 128: return fold_bf16_r<128>(T, D, K, dY, lddy, S, accumulate, ws, st);
    case 256: return fold_bf16_r<256>(T, D, K, dY, lddy, S, accumulate, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
