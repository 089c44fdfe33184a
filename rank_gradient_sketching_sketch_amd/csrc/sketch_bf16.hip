// Sketch accumulation S (+)= dY^T (X A^T), bf16 inputs, on the matrix cores.
//
// The sketch of a weight gradient G = dY^T X is S = G A^T, summed as
// microbatches arrive, so G itself is never formed ("NVIDIA's LoGRA fits RL
// post-training of a 27B model onto a single eight-GPU node", section "Why it
// matters"; "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", paragraph "Gradient sketches."). Two products, both dense
// contractions on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation:
//
//   stage 1   P = c * X Sigma^T  (T x r, contraction over k), this file.
//   stage 2   S (+)= dY^T P  (d x r, contraction over the tokens): the fold
//             kernel in fold_bf16.hip.
//
// Stage 1 design. A workgroup owns 32 tokens (64 where that still gives at
// least 256 workgroups: each sign fragment then feeds four token blocks) x
// 128 (or r, if smaller) sign columns over the whole of k, so no partial sums
// leave the chip: its eight waves (two per SIMD, so one wave's sign
// arithmetic overlaps the other's matrix and memory work) split the k range,
// each accumulating the whole tile, and add their tiles through LDS in a
// fixed order at the end.
// Sigma is never stored: each wave hashes the 64-bit sign words of its k range
// into an LDS table (8 word blocks at a time), and every step expands one byte per lane into
// eight bf16 +-1 values, the B operand of the MFMA. X streams straight from
// HBM through buffer loads (rows past T and columns past k read as zero)
// two steps ahead of use. The result is scaled by c, rounded to bf16
// (nearest even) and written in the fold's operand layout
// P[t / 32][l][t % 32], so a 16-byte load there is one MFMA fragment.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

constexpr int kS1Tokens = 32;     // tokens per P block (the fold's operand layout)
constexpr int kS1Waves = 8;       // waves per workgroup; they split the k range
constexpr int kS1Words = 8;       // sign-word blocks (64 columns of k each) hashed per refill
constexpr int kS1Prefetch = 2;    // steps of X held in registers ahead of use (2 measured
                                  // faster than 4 or 8: every CU requests its X at once)
constexpr int kS1TileBytes = 147456;   // LDS for the reduction tiles (8 waves x 128 x 36 fp32)
constexpr int kS1MinWGs64 = 256;  // workgroups (times the concurrency) from which 64-token ones are used

template <int R>
struct Stage1Shape {
    static constexpr int RT = R < 128 ? R : 128;   // sign columns per workgroup
    static constexpr int NB = RT / 16;             // 16-column MFMA blocks per wave
    static constexpr int NCT = R / RT;             // column tiles
    static_assert(R % 32 == 0 && R <= 256, "bf16 sketch supports r in {32,64,128,256}");
};

// ---------------------------------------------------------------- stage 1 --
// MB 16-row token blocks per workgroup: 2 (32 tokens) or 4 (64 tokens, which
// halves the sign expansion per product where the grid still fills the chip).
template <int R, int MB>
__global__ __launch_bounds__(512) void stage1_bf16_kernel(const uint16_t *__restrict__ X, int64_t ldx,
                                                          int T, int K, uint64_t key, float c,
                                                          uint16_t *__restrict__ P, int p_blocks,
                                                          int *__restrict__ sync, int n_sync) {
    using Sh = Stage1Shape<R>;
    constexpr int RT = Sh::RT, NB = Sh::NB, PF = kS1Prefetch;
    constexpr int TOK = 16 * MB;                       // tokens per workgroup
    constexpr int kTileLd = TOK + 4;                   // fp32 stride of one column of a wave's tile
    constexpr int kWaveTile = RT * kTileLd * 4;        // bytes of one wave's tile
    // wave tiles LDS holds at once: all eight, or four (then waves 4..7 hand
    // theirs to waves 0..3 first)
    constexpr int NT = kS1Waves * kWaveTile <= kS1TileBytes ? kS1Waves : kS1Waves / 2;
    static_assert(NT * kWaveTile <= kS1TileBytes, "reduction tiles exceed the LDS budget");
    constexpr int kTableBytes = kS1Waves * kS1Words * RT * 8;
    constexpr int kTileBytes = NT * kWaveTile;
    // The per-wave sign-word tables during the loop, the reduction tile after it.
    __shared__ __attribute__((aligned(16))) char smem[kTableBytes > kTileBytes ? kTableBytes : kTileBytes];
    uint64_t *table = reinterpret_cast<uint64_t *>(smem);
    float *tile = reinterpret_cast<float *>(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The fold that follows in this workspace starts from zeroed sync words.
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = tid; i < n_sync; i += 64 * kS1Waves) sync[i] = 0;
    const int i16 = lane & 15, g = lane >> 4;
    const int l0 = blockIdx.y * RT;            // first sign column of the tile
    const int t0 = blockIdx.x * TOK;

    // This wave's share of k, in whole 64-column word blocks.
    const int nkb = (K + 63) >> 6;
    const int bpw = (nkb + kS1Waves - 1) / kS1Waves;
    const int kb0 = min(nkb, wave * bpw), kb1 = min(nkb, kb0 + bpw);
    const int s_begin = 2 * kb0;
    const int s_end = min((K + 31) >> 5, 2 * kb1);   // 32-column steps

    // X fragments: lane (i16, g) of row block mb holds X[t0 + 16 mb + i16][32 s + 8 g .. +7].
    constexpr uint32_t kOob = 0x80000000u;
    const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X), 0, static_cast<int>(static_cast<int64_t>(T) * ldx * 2), 0x00020000);
    uint32_t row_off[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int t = t0 + 16 * mb + i16;
        row_off[mb] = t < T ? static_cast<uint32_t>(static_cast<int64_t>(t) * ldx * 2) : kOob;
    }
    auto xload = [&](int s, int mb) -> u32x4_t {
        const int k = 32 * s + 8 * g;
        const uint32_t off = (row_off[mb] != kOob && s < s_end && k < K) ? row_off[mb] + 2u * k : kOob;
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, 0));
    };

    // Sign words of this wave's k range, kS1Words blocks at a time:
    // table[wave][block - first][column].
    uint64_t *wt = table + wave * (kS1Words * RT);
    auto refill = [&](int first) {
        for (int idx = lane; idx < kS1Words * RT; idx += 64) {
            const int bb = idx / RT, col = idx - bb * RT;
            const int b = first + bb;
            wt[idx] = b < kb1 ? sign_word(key, static_cast<uint32_t>(l0 + col), static_cast<uint32_t>(b)) : 0ull;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    };

    f32x4_t acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = zero_f32x4();

    u32x4_t xa[PF][MB];
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xa[p][mb] = xload(s_begin + p, mb);

    const uint32_t one_pair = opaque_u32(0x3F803F80u);   // two bf16 +1.0
    int first = kb0;   // first block held in the table
    if (s_begin < s_end) refill(first);
    // Whole groups of PF steps; steps past s_end load zeros and their
    // (zero) products are skipped.
    for (int s0 = s_begin; s0 < s_end; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            if (s < s_end) {
                const int b = s >> 1;
                if (b >= first + kS1Words) {
                    first += kS1Words;
                    refill(first);
                }
                // B fragments: columns 16 nb + i16, k = 32 s + 8 g .. +7, i.e.
                // byte 4 (s & 1) + g of the word.
                u32x4_t bf[NB];
                const uint64_t *wrow = wt + (b - first) * RT + i16;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const uint64_t w = wrow[16 * nb];
                    const uint32_t dw = (s & 1) ? static_cast<uint32_t>(w >> 32) : static_cast<uint32_t>(w);
                    bf[nb] = signs8_to_bf16(__builtin_amdgcn_ubfe(dw, 8 * g, 8), one_pair);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_bf16(xa[p][mb], bf[nb], acc[mb][nb]);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) xa[p][mb] = xload(s + PF, mb);
        }
    }

    // The waves' tiles go to LDS as tile[wave][column][token] and are added
    // in wave order (with four tiles held at once, wave w + 4 first adds its
    // tile to wave w's, so the sum is (t0 + t4) + (t1 + t5) + ...). Lane
    // (i16, g) of block (mb, nb) holds tokens 16 mb + 4 g .. +3 of column
    // 16 nb + i16.
    __syncthreads();   // every wave is done with its word table
    auto tile_at = [&](int w, int mb, int nb) -> f32x4_t * {
        return reinterpret_cast<f32x4_t *>(&tile[(w * RT + 16 * nb + i16) * kTileLd + 16 * mb + 4 * g]);
    };
    if constexpr (NT < kS1Waves) {
        if (wave >= NT) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) *tile_at(wave - NT, mb, nb) = acc[mb][nb];
        }
        __syncthreads();
        if (wave < NT) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = *tile_at(wave, mb, nb) + acc[mb][nb];
        }
        __syncthreads();
    }
    if (wave < NT) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) *tile_at(wave, mb, nb) = acc[mb][nb];
    }
    __syncthreads();
    // Output chunks: column q / (TOK / 8), tokens 8 (q % (TOK / 8)) .. +7
    // (16 bytes of P), in the P block of those tokens; blocks past the
    // buffer (a ragged last workgroup) are not written.
    constexpr int CPC = TOK / 8;   // chunks per column
    for (int q = tid; q < RT * CPC; q += 64 * kS1Waves) {
        const int col = q / CPC, tq = 8 * (q % CPC);
        const int blk = (t0 + tq) / kS1Tokens;
        if (blk >= p_blocks) continue;
        f32x4_t lo = zero_f32x4(), hi = zero_f32x4();
#pragma unroll
        for (int w = 0; w < NT; ++w) {
            const float *src = &tile[(w * RT + col) * kTileLd + tq];
            lo += *reinterpret_cast<const f32x4_t *>(src);
            hi += *reinterpret_cast<const f32x4_t *>(src + 4);
        }
        u32x4_t o;
        o.x = pack_bf16x2(c * lo.x, c * lo.y);
        o.y = pack_bf16x2(c * lo.z, c * lo.w);
        o.z = pack_bf16x2(c * hi.x, c * hi.y);
        o.w = pack_bf16x2(c * hi.z, c * hi.w);
        *reinterpret_cast<u32x4_t *>(P + (static_cast<size_t>(blk) * R + l0 + col) * kS1Tokens +
                                     (t0 + tq) % kS1Tokens) = o;
    }
}

// ----------------------------------------------------------------- plans --
Stage1Plan plan_stage1_bf16(int64_t T, int64_t K, int R) {
    Stage1Plan p;
    (void)K;
    if (T <= 0) return p;
    p.t_blocks = static_cast<int>((T + kS1Tokens - 1) / kS1Tokens);
    p.col_tiles = R / (R < 128 ? R : 128);
    p.p_bytes = static_cast<size_t>(p.t_blocks) * kS1Tokens * R * 2;
    return p;
}

template <int R>
static hipError_t project_bf16_r(int64_t T, int64_t D, int64_t K, uint64_t key, float c, const uint16_t *X,
                                 int64_t ldx, void *ws, int concurrency, hipStream_t st) {
    const Stage1Plan p = plan_stage1_bf16(T, K, R);
    const FoldPlan f = plan_fold_bf16(T, D, R);
    uint16_t *P = static_cast<uint16_t *>(ws);
    int *sync = reinterpret_cast<int *>(static_cast<char *>(ws) + p.p_bytes + f.xbuf_bytes);
    // 64-token workgroups where they still give a workgroup per compute
    // unit of this call's share of the chip (1 / concurrency of it), and
    // never fewer than half a chip's worth of them (with four streams, 64
    // workgroups of 64 tokens lost to 128 of 32), else 32-token ones
    const int wg64 = (p.t_blocks + 1) / 2;
    const int64_t n64 = static_cast<int64_t>(wg64) * p.col_tiles;
    const bool tall = n64 * concurrency >= kS1MinWGs64 && 2 * n64 >= kS1MinWGs64;
    auto kernel = tall ? stage1_bf16_kernel<R, 4> : stage1_bf16_kernel<R, 2>;
    hipLaunchKernelGGL(kernel, dim3(tall ? wg64 : p.t_blocks, p.col_tiles), dim3(64 * kS1Waves), 0, st, X, ldx,
                       static_cast<int>(T), static_cast<int>(K), key, c, P, p.t_blocks, sync, f.sync_words);
    return hipGetLastError();
}

template <int R>
static hipError_t fold_bf16_r(int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                              float *S, int accumulate, void *ws, const FoldWait &wait, hipStream_t st) {
    const Stage1Plan p = plan_stage1_bf16(T, K, R);
    char *base = static_cast<char *>(ws);
    const uint16_t *P = reinterpret_cast<const uint16_t *>(base);
    void *scratch = base + p.p_bytes;   // exchange buffer, then the sync words
    return launch_fold_bf16_tiles(R, T, D, dY, lddy, P, p.t_blocks, S, accumulate, scratch, wait, st);
}

hipError_t launch_project_bf16(int R, int64_t T, int64_t D, int64_t K, uint64_t key, float c,
                               const uint16_t *X, int64_t ldx, void *ws, int concurrency, hipStream_t st) {
    switch (R) {
    case 32: return project_bf16_r<32>(T, D, K, key, c, X, ldx, ws, concurrency, st);
    case 64: return project_bf16_r<64>(T, D, K, key, c, X, ldx, ws, concurrency, st);
    case 128: return project_bf16_r<128>(T, D, K, key, c, X, ldx, ws, concurrency, st);
    case 256: return project_bf16_r<256>(T, D, K, key, c, X, ldx, ws, concurrency, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fold_parts_ws_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY,
                                     int64_t lddy, float *S, float *parts, int phase, void *ws, hipStream_t st) {
    const Stage1Plan p = plan_stage1_bf16(T, K, R);
    return launch_fold_parts_bf16(R, T, D, dY, lddy, static_cast<const uint16_t *>(ws), p.t_blocks, S, parts,
                                  phase, st);
}

hipError_t launch_fold_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                            float *S, int accumulate, void *ws, const FoldWait &wait, hipStream_t st) {
    switch (R) {
    case 32: return fold_bf16_r<32>(T, D, K, dY, lddy, S, accumulate, ws, wait, st);
    case 64: return fold_bf16_r<64>(T, D, K, dY, lddy, S, accumulate, ws, wait, st);
    case 128: return fold_bf16_r<128>(T, D, K, dY, lddy, S, accumulate, ws, wait, st);
    case 256: return fold_bf16_r<256>(T, D, K, dY, lddy, S, accumulate, ws, wait, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
