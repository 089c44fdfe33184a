// Sketch stage 2 ("fold"): S (+)= dY^T P on the matrix cores, bf16 inputs,
// fp32 accumulation. P = c X Sigma^T is the projected microbatch that stage 1
// left in the workspace; S = G A^T with G = dY^T X is the sketch of the weight
// gradient ("NVIDIA's LoGRA fits RL post-training of a 27B model onto a single
// eight-GPU node", section "Why it matters").
//
// This is the dominant, HBM-bound kernel of the sketch: dY (T x d) is the big
// stream and every byte of it meets all r = 256 columns of P. Design:
//   * One workgroup per compute unit, each owning a contiguous range of 4-5
//     blocks of 16 rows of S (64-80 rows) and all r columns, so dY is read from
//     HBM exactly once and the row ranges are balanced over the 256 CUs. When d
//     is too small to give every CU work, the token range is split as well and
//     a second pass adds the partial tiles in a fixed order.
//   * dY is token-major, but the MFMA wants 8 consecutive tokens per lane. Each
//     thread streams 16-byte chunks of dY rows (8 columns of one token) into a
//     3-slot LDS ring, 4 steps of 32 tokens ahead in registers; the waves then
//     read operand fragments with the gfx950 transpose read ds_read_b64_tr_b16
//     (one 4 x 16 block per 16-lane group, column j to lane j). LDS rows are 80
//     elements (160 bytes) apart, which keeps the four rows of each block on
//     disjoint banks.
//   * P is stored by stage 1 in operand-fragment order, so its fragments come
//     straight from L2 into registers, two steps ahead. The four waves split
//     the r columns (64 each), so no P fragment is read twice in a workgroup.
//   * Barriers wait only for LDS traffic (workgroup fences on the local address
//     space), so the global prefetches stay in flight across them.
#include "common.hpp"
#include "launch.hpp"

namespace logra {

constexpr int kFoldMaxBlocks = 5;     // 16-row blocks per workgroup tile (up to 80 rows)
constexpr int kFoldLdsRow = 80;       // bf16 elements per LDS row of a ring slot
constexpr int kFoldSlots = 3;         // LDS ring slots (one step of 32 tokens each)
constexpr int kFoldPrefetch = 8;      // steps of dY held in registers ahead of use
constexpr int kXcds = 8;              // gfx950: workgroup ids go round-robin over 8 XCDs
constexpr int kFoldTargetWGs = 256;   // one workgroup per compute unit

template <int R>
struct FoldShape {
    static constexpr int NB = R / 16;            // 16-wide column blocks of r
    static constexpr int WN = NB < 4 ? NB : 4;   // waves across r
    static constexpr int NBW = NB / WN;          // column blocks per wave
    static constexpr int WM = 4 / WN;            // waves across row blocks
    static constexpr int MBW = (kFoldMaxBlocks + WM - 1) / WM;   // row blocks per wave (max)
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Transposed LDS read: each 16-lane group supplies the addresses of a 4 x 16
// block of bf16 (lane i: row i/4, columns 4*(i%4) .. +3) and lane j receives
// column j (rows 0..3).
__device__ __forceinline__ u32x2_t lds_read_tr(const uint16_t *p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
    return __builtin_bit_cast(u32x2_t, v);
}

// Barrier that orders LDS traffic only (global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int R>
__global__ __launch_bounds__(256) void fold_bf16_kernel(
    const uint16_t *__restrict__ dY, int64_t lddy, int T, int D, const uint16_t *__restrict__ P,
    int p_blocks, float *__restrict__ S, float *__restrict__ part, int accumulate, int nblk,
    int n_wg_d, int steps_per) {
    using Sh = FoldShape<R>;
    constexpr int NBW = Sh::NBW, MBW = Sh::MBW, WM = Sh::WM, PF = kFoldPrefetch;
    constexpr int kSlot = 32 * kFoldLdsRow;             // one step: 32 token rows
    constexpr int kTileRows = kFoldMaxBlocks * 16;      // rows of S per workgroup (max)
    constexpr int kTileLd = R + 4;                      // fp32 row stride of the output tile in LDS
    constexpr int kRowChunks = R / 4;                   // 16-byte chunks per row of S
    constexpr int kOutChunks = (kTileRows * kRowChunks + 255) / 256;   // per thread
    constexpr int kRingBytes = kFoldSlots * kSlot * 2;
    constexpr int kTileBytes = kTileRows * kTileLd * 4;
    // The dY ring during the loop, the output tile in the epilogue.
    __shared__ __attribute__((aligned(16))) char smem[kRingBytes > kTileBytes ? kRingBytes : kTileBytes];
    uint16_t *lds = reinterpret_cast<uint16_t *>(smem);
    float *tile = reinterpret_cast<float *>(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index as a scalar: every per-wave decision below is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Sh::WN, wn = wave % Sh::WN;
    const int i16 = lane & 15, g = lane >> 4;
    const int sp = blockIdx.y;
    // Consecutive row tiles go to the same XCD (ids are dealt round-robin over
    // the XCDs), so the cache lines two neighbouring tiles share are fetched
    // into one L2 only.
    const int wg = (n_wg_d % kXcds == 0)
                       ? (blockIdx.x % kXcds) * (n_wg_d / kXcds) + blockIdx.x / kXcds
                       : static_cast<int>(blockIdx.x);
    const int b0 = static_cast<int>((static_cast<int64_t>(wg) * nblk) / n_wg_d);
    const int b1 = static_cast<int>((static_cast<int64_t>(wg + 1) * nblk) / n_wg_d);
    const int nmb = b1 - b0;
    const int d0 = b0 * 16;
    const int cpr = nmb * 2;              // 16-byte chunks per token row of the tile
    const int nchunk = 32 * cpr;          // chunks per step of 32 tokens
    const int nsteps = (T + 31) >> 5;
    const int s_begin = sp * steps_per;
    const int s_end = min(nsteps, s_begin + steps_per);
    const int l_base = wn * NBW * 16;

    // Buffer views: loads past num_records return zero and stores there are
    // dropped, which masks the token tail, the phantom steps after s_end,
    // rows past d and every access sent to kOob.
    constexpr uint32_t kOob = 0x80000000u;
    const __amdgpu_buffer_rsrc_t dy_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(dY), 0, static_cast<int>(static_cast<int64_t>(T) * lddy * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(P), 0, static_cast<int>(static_cast<int64_t>(p_blocks) * R * 64),
        0x00020000);
    float *dst = part ? part + static_cast<size_t>(sp) * D * R : S;
    const __amdgpu_buffer_rsrc_t s_rs =
        __builtin_amdgcn_make_buffer_rsrc(dst, 0, static_cast<int>(static_cast<int64_t>(D) * R * 4), 0x00020000);

    // The (at most two) 16-byte dY chunks this thread moves per step. Chunk
    // counts are multiples of 64, so whether a wave has a chunk is uniform
    // across the wave.
    const bool has[2] = {wave * 64 < nchunk, wave * 64 + 256 < nchunk};
    uint32_t q_goff[2];   // byte offset of the chunk in token row 0
    int q_loff[2];        // element offset in a slot
    bool q_ok[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = tid + 256 * k;
        const bool on = q < nchunk;
        const int t = on ? q / cpr : 0;
        const int c = on ? q - t * cpr : 0;
        q_ok[k] = on && d0 + 8 * c < D;
        q_goff[k] = static_cast<uint32_t>((static_cast<int64_t>(t) * lddy + d0 + 8 * c) * 2);
        q_loff[k] = t * kFoldLdsRow + 8 * c;
    }
    const uint32_t row_step_bytes = static_cast<uint32_t>(lddy * 2 * 32);   // one step of 32 tokens
    auto gload = [&](int s, int k) -> u32x4_t {
        const uint32_t off = (q_ok[k] && s < s_end) ? q_goff[k] + static_cast<uint32_t>(s) * row_step_bytes
                                                   : kOob;
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(dy_rs, off, 0, 0));
    };
    auto lstore = [&](int s, const u32x4_t &v, int k) {
        if (has[k]) *reinterpret_cast<u32x4_t *>(&lds[(s % kFoldSlots) * kSlot + q_loff[k]]) = v;
    };
    auto bload = [&](int s, u32x4_t (&b)[NBW]) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int l = l_base + 16 * nb + i16;
            const uint32_t off = s < s_end ? static_cast<uint32_t>(((s * R + l) * 32 + 8 * g) * 2) : kOob;
            b[nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(p_rs, off, 0, 0));
        }
    };
    auto aread = [&](int s, u32x4_t (&a)[MBW]) {
        const uint16_t *base = &lds[(s % kFoldSlots) * kSlot];
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            // blocks past this tile read stale LDS; their products are never stored
            const int mb = wm + j * WM;
            const uint16_t *p = base + (8 * g + (i16 >> 2)) * kFoldLdsRow + 16 * mb + 4 * (i16 & 3);
            const u32x2_t lo = lds_read_tr(p);
            const u32x2_t hi = lds_read_tr(p + 4 * kFoldLdsRow);
            a[j] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
    };
    // Output chunk c of this thread: row (tid + 256 c) / kRowChunks of the
    // tile, 4 columns from 4 * ((tid + 256 c) % kRowChunks).
    auto out_off = [&](int c) -> uint32_t {
        const int q = tid + 256 * c;
        const int row = q / kRowChunks, col = 4 * (q % kRowChunks);
        return row < nmb * 16 ? static_cast<uint32_t>(((d0 + row) * R + col) * 4) : kOob;
    };

    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int j = 0; j < MBW; ++j)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[j][nb] = zero_f32x4();

    // Prefetch ring: dY chunks and P fragments of the next PF steps, issued
    // in step order, so that every wait below is for a load issued PF - 1 or
    // PF steps earlier (loads complete in issue order).
    u32x4_t raw[PF][2];
    u32x4_t pb[PF][NBW];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
        for (int k = 0; k < 2; ++k) raw[p][k] = gload(s_begin + p, k);
        bload(s_begin + p, pb[p]);
    }
    // The old S tile, read while the stream runs (the first waits are for
    // the loads above, issued before these).
    const bool add_old = accumulate && !part;
    u32x4_t old[kOutChunks];
#pragma unroll
    for (int c = 0; c < kOutChunks; ++c)
        old[c] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s_rs, add_old ? out_off(c) : kOob, 0, 0));

    u32x4_t a_cur[MBW], a_nxt[MBW];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        lstore(s_begin, raw[0][k], k);
        raw[0][k] = gload(s_begin + PF, k);
    }
    lds_barrier();
    aread(s_begin, a_cur);

    // Whole groups of PF steps; up to PF-1 steps past s_end load zeros and
    // add nothing.
    for (int s0 = s_begin; s0 < s_end; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            // raw[(p + 1) % PF] holds the dY of step s + 1 and pb[p] the P
            // fragments of step s (s0 - s_begin is a multiple of PF)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                lstore(s + 1, raw[(p + 1) % PF][k], k);
                raw[(p + 1) % PF][k] = gload(s + 1 + PF, k);
            }
            lds_barrier();
            aread(s + 1, a_nxt);
#pragma unroll
            for (int j = 0; j < MBW; ++j) {
                if (wm + j * WM < nmb) {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        acc[j][nb] = mfma_bf16(a_cur[j], pb[p][nb], acc[j][nb]);
                }
            }
            bload(s + PF, pb[p]);
#pragma unroll
            for (int j = 0; j < MBW; ++j) a_cur[j] = a_nxt[j];
        }
    }

    // Epilogue: the accumulators go through LDS into row-major order, so that
    // the read-modify-write of S is whole 16-byte chunks of rows. Lane
    // (i16, g) of row block mb holds rows 16 mb + 4 g + e, column
    // l_base + 16 nb + i16.
    lds_barrier();   // every wave is done with the ring
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        const int mb = wm + j * WM;
        if (mb < nmb) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    tile[(16 * mb + 4 * g + e) * kTileLd + l_base + 16 * nb + i16] = acc[j][nb][e];
        }
    }
    lds_barrier();
#pragma unroll
    for (int c = 0; c < kOutChunks; ++c) {
        const int q = tid + 256 * c;
        const int row = min(q / kRowChunks, kTileRows - 1), col = 4 * (q % kRowChunks);
        f32x4_t v = *reinterpret_cast<const f32x4_t *>(&tile[row * kTileLd + col]);
        if (add_old) v += __builtin_bit_cast(f32x4_t, old[c]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), s_rs, out_off(c), 0, 0);
    }
}

// S = [S +] (part_0 + part_1 + ...), token splits added in order.
__global__ __launch_bounds__(256) void fold_reduce_kernel(const float *__restrict__ part, int n_split,
                                                          int64_t n, float *__restrict__ S,
                                                          int accumulate) {
    const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (idx >= n) return;
    f32x4_t t = *reinterpret_cast<const f32x4_t *>(part + idx);
    for (int sp = 1; sp < n_split; ++sp) t += *reinterpret_cast<const f32x4_t *>(part + sp * n + idx);
    f32x4_t *dst = reinterpret_cast<f32x4_t *>(S + idx);
    if (accumulate) t = *dst + t;
    *dst = t;
}

FoldPlan plan_fold_bf16(int64_t T, int64_t D, int R) {
    FoldPlan p;
    if (T <= 0) return p;
    p.nblk = static_cast<int>((D + 15) / 16);
    const int nsteps = static_cast<int>((T + 31) / 32);
    if (p.nblk >= kFoldTargetWGs * 4) {
        p.n_wg_d = p.nblk > kFoldTargetWGs * kFoldMaxBlocks
                       ? (p.nblk + kFoldMaxBlocks - 1) / kFoldMaxBlocks
                       : kFoldTargetWGs;
        p.n_split = 1;
    } else {
        p.n_wg_d = (p.nblk + 3) / 4;
        int ns = kFoldTargetWGs / p.n_wg_d;
        // keep the partial tiles no larger than the dY they replace, and at
        // least 4 steps per split
        const int64_t cap_bytes = T / (2 * R);
        if (ns > cap_bytes) ns = static_cast<int>(cap_bytes);
        if (ns > nsteps / 4) ns = nsteps / 4;
        if (ns < 1) ns = 1;
        p.n_split = ns;
    }
    p.steps_per = (nsteps + p.n_split - 1) / p.n_split;
    p.n_split = (nsteps + p.steps_per - 1) / p.steps_per;
    p.part_bytes = p.n_split > 1 ? static_cast<size_t>(p.n_split) * D * R * 4 : 0;
    return p;
}

template <int R>
static hipError_t fold_r(int64_t T, int64_t D, const uint16_t *dY, int64_t lddy, const uint16_t *P,
                         int p_blocks, float *S, int accumulate, float *part, hipStream_t st) {
    const FoldPlan p = plan_fold_bf16(T, D, R);
    float *dst_part = p.n_split > 1 ? part : nullptr;
    hipLaunchKernelGGL(fold_bf16_kernel<R>, dim3(p.n_wg_d, p.n_split), dim3(256), 0, st, dY, lddy,
                       static_cast<int>(T), static_cast<int>(D), P, p_blocks, S, dst_part, accumulate, p.nblk,
                       p.n_wg_d, p.steps_per);
    if (p.n_split > 1) {
        const int64_t n = D * R;
        hipLaunchKernelGGL(fold_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, part,
                           p.n_split, n, S, accumulate);
    }
    return hipGetLastError();
}

hipError_t launch_fold_bf16_tiles(int R, int64_t T, int64_t D, const uint16_t *dY, int64_t lddy,
                                  const uint16_t *P, int p_blocks, float *S, int accumulate,
                                  float *part, hipStream_t st) {
    switch (R) {
    case 32: return fold_r<32>(T, D, dY, lddy, P, p_blocks, S, accumulate, part, st);
    case 64: return fold_r<64>(T, D, dY, lddy, P, p_blocks, S, accumulate, part, st);
    case 128: return fold_r<128>(T, D, dY, lddy, P, p_blocks, S, accumulate, part, st);
    case 256: return fold_r<256>(T, D, dY, lddy, P, p_blocks, S, accumulate, part, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
