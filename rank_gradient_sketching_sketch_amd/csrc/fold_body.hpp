// The body of the sketch's fold, S (+)= dY^T P, for one workgroup: shared
// by the fold kernel (fold_bf16.hip) and the backward kernel that runs it
// beside the dX product (dx_bf16.hip). The design is described at the top of
// fold_bf16.hip.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace logra {

constexpr int kFoldSlots = 3;         // LDS ring slots (one step of 32 tokens each)
constexpr int kFoldMaxSplit = 32;     // members per tile (most)
constexpr int kXcds = 8;              // gfx950: workgroup ids go round-robin over 8 XCDs
constexpr int kFoldWGs = 256;         // one workgroup per compute unit

// Shape of one kernel instance. MAXB (5 or 10) bounds the 16-row blocks of a
// tile; tiles are planned to hold MAXB or MAXB - 1 blocks where d allows,
// and the waves compute every block but the last unconditionally (products
// of blocks past the tile are never stored), which keeps the unrolled steps
// free of branches.
template <int R, int MAXB, int STAGE_ROWS = (R >= 256 ? 80 : 160)>
struct FoldShape {
    static constexpr int NB = R / 16;            // 16-wide column blocks of r
    static constexpr int WN = NB < 4 ? NB : 4;   // waves across r
    static constexpr int NBW = NB / WN;          // column blocks per wave
    static constexpr int WM = 4 / WN;            // waves across row blocks
    static constexpr int MBW = (MAXB + WM - 1) / WM;   // row blocks per wave
    static constexpr int LDS_ROW = 16 * MAXB;    // bf16 elements per LDS token row of a ring slot
    static constexpr int NCH = (32 * 2 * MAXB + 255) / 256;   // dY chunks per thread per step
    static constexpr int PF = MAXB > 5 ? 4 : 8;  // steps of dY and P held in registers ahead of use
    static constexpr int HALF = (MBW + 1) / 2;   // a wave's row blocks finalized by the first of two members
    static constexpr int STAGE = STAGE_ROWS;             // rows of the epilogue staging tile
    static constexpr int RING_BYTES = 3 * 32 * LDS_ROW * 2;             // the dY ring (kFoldSlots steps)
    static constexpr int TILE_BYTES = STAGE * (R + 4) * 4;              // the epilogue staging tile
    static constexpr int LDS_BYTES = RING_BYTES > TILE_BYTES ? RING_BYTES : TILE_BYTES;
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

// Cache policies of the exchange traffic. Between XCDs: device scope (the
// SC1 bit, what agent-scope atomic loads and stores compile to on gfx950), so
// a partial written on one XCD is read correctly from another. Within one
// XCD the shared L2 is the point of coherence: plain stores (the vector L1
// writes through) and loads that bypass the L1 (SC0, workgroup scope).
constexpr int kDeviceScope = 16;
constexpr int kL1Bypass = 1;
// s_getreg operand of HW_REG_XCC_ID (register 20, bits 0..3): the XCD a wave runs on.
constexpr int kHwRegXccId = 20 | (0 << 6) | (3 << 11);

// How the members of a tile add their partials: one member (nothing to
// add); two, exchanging MFMA fragments within the kernel; more, each
// writing its partial tile for fold_reduce_kernel to add; or split: the
// sketch is kept in parts across the microbatches of a step, member 0 adding
// its partial to S and member q > 0 to part q - 1 (xbuf + (q - 1) d r), with
// no exchange and no waiting inside the kernel.
enum FoldMode { kFoldSingle = 0, kFoldPair = 1, kFoldPartial = 2, kFoldSplit = 3 };

// The fold of one workgroup. smem (FoldShape::LDS_BYTES, 16-byte aligned) and
// s_word are the caller's LDS; fixed_ticket >= 0 names the workgroup's tile
// and member directly (single mode, used when the fold shares a launch with
// other work), otherwise they come from the workgroup id (or, in pair mode,
// from the ticket counter).
template <int R, int MAXB, int MODE, int STAGE_ROWS = (R >= 256 ? 80 : 160)>
__device__ __forceinline__ void fold_body(
    char *smem, int &s_word, int fixed_ticket,
    const uint16_t *__restrict__ dY, int64_t lddy, int T, int D, const uint16_t *__restrict__ P,
    int p_blocks, float *__restrict__ S, float *__restrict__ xbuf, int x_bytes, int *__restrict__ sync,
    int accumulate, int nblk, int n_tiles, int n_split, int steps_per, int spin_limit, int *__restrict__ timeouts) {
    using Sh = FoldShape<R, MAXB, STAGE_ROWS>;
    constexpr int NBW = Sh::NBW, MBW = Sh::MBW, WM = Sh::WM, PF = Sh::PF, NCH = Sh::NCH;
    constexpr int kLdsRow = Sh::LDS_ROW;
    constexpr int kSlot = 32 * kLdsRow;                 // one step: 32 token rows
    constexpr int kTileLd = R + 4;                      // fp32 row stride of the staging tile in LDS
    constexpr int kRowChunks = R / 4;                   // 16-byte chunks per row of S
    constexpr int kStage = Sh::STAGE;
    constexpr int kOutChunks = (kStage * kRowChunks + 255) / 256;   // per thread per staged pass
    static_assert(Sh::RING_BYTES == kFoldSlots * kSlot * 2, "ring size");
    // The dY ring during the loop, the staging tile in the epilogue.
    uint16_t *lds = reinterpret_cast<uint16_t *>(smem);
    float *tile = reinterpret_cast<float *>(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index as a scalar: every per-wave decision below is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Sh::WN, wn = wave % Sh::WN;
    const int i16 = lane & 15, g = lane >> 4;
    const int G = n_tiles * n_split;

    // Sync words of the pair mode: the ticket counter, one counter per id
    // group, each member's flag, each tile's done count, each member's XCD.
    int *flags = sync + 1 + kXcds;
    int *done = flags + G;
    int *xcd_of = done + n_tiles;
    // Tile and member: a ticket when members exchange partials; otherwise
    // the workgroup id, with consecutive tiles on one XCD (ids are dealt
    // round-robin over the XCDs) so the cache lines that neighbouring tiles
    // share are fetched into one L2.
    int ticket;
    if (fixed_ticket >= 0) {
        ticket = fixed_ticket;
    } else if (MODE == kFoldPair) {
        if (tid == 0) {
            // With G a multiple of 16, the ids of one group (id mod 8, the
            // XCD they are dealt to) draw tickets among themselves and hold
            // consecutive tiles, so a tile's two members and its neighbours
            // normally share an XCD; otherwise one counter for all.
            const bool grouped = G % (2 * kXcds) == 0;
            const int grp = static_cast<int>(blockIdx.x % kXcds);
            int *ctr = grouped ? sync + 1 + grp : sync;
            const int n = grouped ? G / kXcds : G;
            const unsigned t = static_cast<unsigned>(
                __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            // in range even if the counter was not zeroed (no projection made
            // in this workspace): then the results are undefined, not a fault
            const int lt = static_cast<int>(t % static_cast<unsigned>(n));
            if (lt == n - 1) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int tk = grouped ? grp * n + lt : lt;
            // the XCD this workgroup runs on (hardware register), published
            // for the partner as id + 1
            const int xcd = static_cast<int>(__builtin_amdgcn_s_getreg(kHwRegXccId) & 15u);
            __hip_atomic_store(xcd_of + tk, xcd + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_word = tk;
        }
        __syncthreads();
        ticket = __builtin_amdgcn_readfirstlane(s_word);
    } else {
        ticket = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds
                                  : static_cast<int>(blockIdx.x);
    }
    const int ti = ticket / n_split, mem = ticket % n_split;
    const int b0 = static_cast<int>((static_cast<int64_t>(ti) * nblk) / n_tiles);
    const int b1 = static_cast<int>((static_cast<int64_t>(ti + 1) * nblk) / n_tiles);
    const int nmb = b1 - b0;
    const int d0 = b0 * 16;
    const int rows = nmb * 16;
    const int cpr = nmb * 2;              // 16-byte chunks per token row of the tile
    const int nchunk = 32 * cpr;          // chunks per step of 32 tokens
    const int nsteps = (T + 31) >> 5;
    const int s_begin = min(nsteps, mem * steps_per);
    const int s_end = min(nsteps, s_begin + steps_per);
    const int l_base = wn * NBW * 16;

    // Rows this member finalizes: with two members, the first finalizes the
    // first HALF row blocks of every wave (rows [0, 16 WM HALF)) and the
    // second the rest, and their partials move as MFMA fragments (1 KB per
    // wave and block, no staging); with more members, consecutive row ranges,
    // and the partials move as rows.
    constexpr int kHalf = Sh::HALF;
    static_assert(MODE != kFoldPair || 16 * WM * (MBW - kHalf > kHalf ? MBW - kHalf : kHalf) <= kStage,
                  "each member of a pair finalizes its rows in one staged pass");
    int own0, own1;
    if (MODE == kFoldPair) {
        own0 = mem == 0 ? 0 : min(16 * WM * kHalf, rows);
        own1 = mem == 0 ? min(16 * WM * kHalf, rows) : rows;
    } else {
        own0 = 0;
        own1 = MODE == kFoldSingle || MODE == kFoldSplit ? rows : 0;
    }


    // Buffer views: loads past num_records return zero and stores there are
    // dropped, which masks the token tail, the phantom steps after s_end,
    // rows past d and every access sent to kOob.
    constexpr uint32_t kOob = 0x80000000u;
    const __amdgpu_buffer_rsrc_t dy_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(dY), 0, static_cast<int>(static_cast<int64_t>(T) * lddy * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(P), 0, static_cast<int>(static_cast<int64_t>(p_blocks) * R * 64),
        0x00020000);
    // the member's share of the sketch: S, or in split mode its part
    float *dst = MODE == kFoldSplit && mem > 0 ? xbuf + static_cast<int64_t>(mem - 1) * D * R : S;
    const __amdgpu_buffer_rsrc_t s_rs =
        __builtin_amdgcn_make_buffer_rsrc(dst, 0, static_cast<int>(static_cast<int64_t>(D) * R * 4), 0x00020000);

    // The (up to NCH) 16-byte dY chunks this thread moves per step. Chunk
    // counts are multiples of 64, so whether a wave has a chunk is uniform
    // across the wave.
    bool has[NCH];
    uint32_t q_goff[NCH];   // byte offset of the chunk in token row 0
    int q_loff[NCH];        // element offset in a slot
    bool q_ok[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int q = tid + 256 * k;
        has[k] = wave * 64 + 256 * k < nchunk;
        const bool on = q < nchunk;
        const int t = on ? q / cpr : 0;
        const int c = on ? q - t * cpr : 0;
        q_ok[k] = on && d0 + 8 * c < D;
        q_goff[k] = static_cast<uint32_t>((static_cast<int64_t>(t) * lddy + d0 + 8 * c) * 2);
        q_loff[k] = t * kLdsRow + 8 * c;
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
    // every block but the last is read whatever the tile height (stale LDS
    // past the tile feeds products that are never stored)
    auto aread = [&](int s, u32x4_t (&a)[MBW]) {
        const uint16_t *base = &lds[(s % kFoldSlots) * kSlot];
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            const int mb = wm + j * WM;
            if (j < MBW - 1 || mb < nmb) {
                const uint16_t *p = base + (8 * g + (i16 >> 2)) * kLdsRow + 16 * mb + 4 * (i16 & 3);
                const u32x2_t lo = lds_read_tr(p);
                const u32x2_t hi = lds_read_tr(p + 4 * kLdsRow);
                a[j] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
            }
        }
    };

    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int j = 0; j < MBW; ++j)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[j][nb] = zero_f32x4();

    // Prefetch ring: dY chunks and P fragments of the next PF steps, issued
    // in step order, so that every wait below is for a load issued PF - 1 or
    // PF steps earlier (loads complete in issue order).
    u32x4_t raw[PF][NCH];
    u32x4_t pb[PF][NBW];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) raw[p][k] = gload(s_begin + p, k);
        bload(s_begin + p, pb[p]);
    }

    // dY^T fragments, double-buffered by step parity (PF is even, so the
    // buffer of a step is a compile-time index and nothing is copied)
    static_assert(PF % 2 == 0, "an even prefetch depth keeps the fragment buffers fixed");
    u32x4_t afr[2][MBW];
#pragma unroll
    for (int j = 0; j < MBW; ++j) afr[0][j] = afr[1][j] = zero_u32x4();
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        lstore(s_begin, raw[0][k], k);
        raw[0][k] = gload(s_begin + PF, k);
    }
    lds_barrier();
    aread(s_begin, afr[0]);

    // Whole groups of PF steps; up to PF-1 steps past s_end load zeros and
    // add nothing.
    for (int s0 = s_begin; s0 < s_end; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int s = s0 + p;
            // raw[(p + 1) % PF] holds the dY of step s + 1 and pb[p] the P
            // fragments of step s (s0 - s_begin is a multiple of PF)
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                lstore(s + 1, raw[(p + 1) % PF][k], k);
                raw[(p + 1) % PF][k] = gload(s + 1 + PF, k);
            }
            lds_barrier();
            aread(s + 1, afr[(p + 1) % 2]);
#pragma unroll
            for (int j = 0; j < MBW; ++j) {
                if (j < MBW - 1 || wm + j * WM < nmb) {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        acc[j][nb] = mfma_bf16(afr[p % 2][j], pb[p][nb], acc[j][nb]);
                }
            }
            bload(s + PF, pb[p]);
        }
    }

    // ---- epilogue. The accumulators go through LDS into row-major order in
    // passes of up to kStage rows, so that S moves in whole 16-byte row
    // chunks. Lane (i16, g) of row block mb holds rows 16 mb + 4 g + e,
    // column l_base + 16 nb + i16.

    // stage rows [r0, r1) of the tile
    auto stage = [&](int r0, int r1) {
        lds_barrier();   // the previous user of the LDS is done
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            const int mb = wm + j * WM;
            if (mb < nmb && 16 * mb + 16 > r0 && 16 * mb < r1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * mb + 4 * g + e;
                    if (row >= r0 && row < r1) {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            tile[(row - r0) * kTileLd + l_base + 16 * nb + i16] = acc[j][nb][e];
                    }
                }
            }
        }
        lds_barrier();
    };
    // Chunk c of this thread in a pass from row r0: tile row
    // r0 + (tid + 256 c) / kRowChunks, columns 4 ((tid + 256 c) % kRowChunks) .. +3.
    auto chunk_row = [&](int r0, int c) { return r0 + (tid + 256 * c) / kRowChunks; };
    auto chunk_col = [&](int c) { return 4 * ((tid + 256 * c) % kRowChunks); };
    auto staged = [&](int r0, int c) -> f32x4_t {
        const int lr = min(chunk_row(r0, c) - r0, kStage - 1);
        return *reinterpret_cast<const f32x4_t *>(&tile[lr * kTileLd + chunk_col(c)]);
    };
    // byte offset of (tile row, column) in a d x r fp32 matrix
    auto s_off = [&](int row, int col) -> uint32_t {
        return static_cast<uint32_t>(((d0 + row) * R + col) * 4);
    };
    // byte offset of chunk c of a pass over rows [r0, r1) in a d x r matrix (kOob outside)
    auto c_off = [&](int r0, int r1, int c) -> uint32_t {
        const int row = chunk_row(r0, c);
        return (row < r1 && d0 + row < D) ? s_off(row, chunk_col(c)) : kOob;
    };

    const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(xbuf, 0, x_bytes, 0x00020000);
    const uint32_t x_stride = static_cast<uint32_t>(static_cast<int64_t>(D) * R * 4);   // rows layout
    // fragment (member q, row block mb, column block nb of this wave) in the
    // fragment layout: 1 KB per wave, 16 bytes per lane
    auto x_frag = [&](int q, int mb, int nb) -> uint32_t {
        return static_cast<uint32_t>(((((ti * 2 + q) * MAXB + mb) * Sh::WN + wn) * NBW + nb) * 1024 + lane * 16);
    };

    // Old values of the rows a member of a pair finalizes (a single pass):
    // requested before the exchange stores, so both drain together.
    u32x4_t old_pre[kOutChunks];
    bool same_xcd = false;   // the pair's exchange stays in one L2
    if (MODE == kFoldPair) {
#pragma unroll
        for (int c = 0; c < kOutChunks; ++c)
            old_pre[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         s_rs, accumulate ? c_off(own0, own1, c) : kOob, 0, 0));
        // whether the other member runs on this XCD (it has published its
        // XCD since it started; a bounded wait, as for its flag below)
        if (tid == 0) {
            const int mine = static_cast<int>(__builtin_amdgcn_s_getreg(kHwRegXccId) & 15u) + 1;
            int other = 0;
            for (int spins = 0; spins <= spin_limit; ++spins) {
                other = __hip_atomic_load(xcd_of + ti * n_split + (1 - mem), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                if (other != 0) break;
                __builtin_amdgcn_s_sleep(1);
            }
            s_word = other == mine;
        }
        __syncthreads();
        same_xcd = s_word != 0;
        // 1. this member's fragments of the blocks the other finalizes,
        // straight from the accumulators
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            const int mb = wm + j * WM;
            if (mb < nmb && (j < kHalf) == (mem == 1)) {
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const u32x4_t v = __builtin_bit_cast(u32x4_t, acc[j][nb]);
                    if (same_xcd)
                        __builtin_amdgcn_raw_buffer_store_b128(v, x_rs, x_frag(mem, mb, nb), 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b128(v, x_rs, x_frag(mem, mb, nb), 0, kDeviceScope);
                }
            }
        }
    } else if (MODE == kFoldPartial) {
        // this member's partial of the whole tile, for fold_reduce_kernel
        for (int r0 = 0; r0 < rows; r0 += kStage) {
            const int r1 = min(r0 + kStage, rows);
            stage(r0, r1);
#pragma unroll
            for (int c = 0; c < kOutChunks; ++c) {
                const uint32_t off = c_off(r0, r1, c);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, staged(r0, c)), x_rs,
                                                      off == kOob ? kOob : off + mem * x_stride, 0, 0);
            }
        }
        return;
    }
    if (MODE == kFoldPair) {
        // 2. raise the flag: the barrier orders every thread's fragment stores
        // before thread 0's agent-scope release, which makes them visible to
        // the other member wherever it runs
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(flags + ti * n_split + mem, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 3. finalize the own rows, in passes of up to kStage rows (a single pass
    // whenever n_split > 1): add the other members' partials, stage, then
    // read-modify-write S. Without an exchange and with at most two passes,
    // the old values of both passes are requested before the first is
    // staged, so the second pass does not wait for its loads (with the short
    // staging tile of the backward kernel's fold, five passes, they would
    // not fit in its registers).
    constexpr int kPasses = (16 * MAXB + kStage - 1) / kStage;
    constexpr bool kEarlyOld = MODE != kFoldPair && kPasses <= 2;
    u32x4_t old_all[kEarlyOld ? kPasses : 1][kOutChunks];
    if (kEarlyOld) {
#pragma unroll
        for (int q = 0; q < kPasses; ++q) {
            const int q0 = own0 + q * kStage, q1 = min(q0 + kStage, own1);
#pragma unroll
            for (int c = 0; c < kOutChunks; ++c)
                old_all[q][c] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                 s_rs, accumulate && q0 < own1 ? c_off(q0, q1, c) : kOob, 0, 0));
        }
    }
    // (unrolled where the old values were requested early, so that the index
    // into them is a constant)
    constexpr int kUnroll = kEarlyOld ? kPasses : 1;
#pragma unroll kUnroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int r0 = own0 + pass * kStage;
        if (r0 >= own1) break;
        const int r1 = min(r0 + kStage, own1);
        bool timed_out = false;
        if (MODE == kFoldPair) {
            // wait for the other members' partials
            if (tid == 0) {
                int ok = 1;
                for (int q = 0; q < n_split && ok; ++q) {
                    if (q == mem) continue;
                    if (spin_limit < 0) {
                        ok = 0;
                        break;
                    }
                    int spins = 0;
                    while (__hip_atomic_load(flags + ti * n_split + q, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == 0) {
                        if (++spins > spin_limit) {
                            ok = 0;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                if (ok) {
                    // the other member's fragments, released with its flag,
                    // are visible to every load that follows
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                } else if (timeouts) {
                    __hip_atomic_fetch_add(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                s_word = ok;
            }
            __syncthreads();
            timed_out = s_word == 0;
        }
        // S = [S +] v for the chunks of the pass, the old S loads all in flight
        // first (unless the staged values already hold it)
        auto finish_all = [&](auto &&value, bool add_old) {
            u32x4_t old[kOutChunks];
#pragma unroll
            for (int c = 0; c < kOutChunks; ++c)
                old[c] = MODE == kFoldPair ? old_pre[c]
                         : kEarlyOld       ? old_all[kEarlyOld ? pass : 0][c]
                                           : __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                             s_rs, add_old ? c_off(r0, r1, c) : kOob, 0, 0));
#pragma unroll
            for (int c = 0; c < kOutChunks; ++c) {
                f32x4_t v = value(c);
                if (add_old) v = __builtin_bit_cast(f32x4_t, old[c]) + v;
                if (timed_out)
                    v = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), s_rs, c_off(r0, r1, c), 0, 0);
            }
        };
        if (MODE == kFoldPair) {
            // the other member's fragments of the own blocks, all in flight
            // before they are added during staging; part_0 + part_1 is the
            // same sum whichever member adds it
            auto pair = [&](auto j0c, auto j1c) {
                constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
                f32x4_t x[kHalf][NBW];
#pragma unroll
                for (int j = J0; j < J1; ++j) {
                    const int mb = wm + j * WM;
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const uint32_t off = mb < nmb ? x_frag(1 - mem, mb, nb) : kOob;
                        x[j - J0][nb] = __builtin_bit_cast(
                            f32x4_t, same_xcd ? __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, kL1Bypass)
                                              : __builtin_amdgcn_raw_buffer_load_b128(x_rs, off, 0, kDeviceScope));
                    }
                }
                // stage the own rows (all of blocks J0 .. J1 - 1) as acc + x
                lds_barrier();   // the previous user of the LDS is done
#pragma unroll
                for (int j = J0; j < J1; ++j) {
                    const int mb = wm + j * WM;
                    if (mb < nmb) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = 16 * mb + 4 * g + e;
#pragma unroll
                            for (int nb = 0; nb < NBW; ++nb)
                                tile[(row - r0) * kTileLd + l_base + 16 * nb + i16] =
                                    acc[j][nb][e] + x[j - J0][nb][e];
                        }
                    }
                }
                lds_barrier();
            };
            if (mem == 0)
                pair(std::integral_constant<int, 0>{}, std::integral_constant<int, kHalf>{});
            else
                pair(std::integral_constant<int, kHalf>{}, std::integral_constant<int, MBW>{});
            finish_all([&](int c) { return staged(r0, c); }, accumulate != 0);
        } else {
            stage(r0, r1);
            finish_all([&](int c) { return staged(r0, c); }, accumulate != 0);
        }
    }

    if (MODE == kFoldPair) {
        // 4. the last member of the tile to finish clears the tile's flags
        // for the next fold (no member polls them any more)
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(done + ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (prev == n_split - 1) {
                for (int q = 0; q < n_split; ++q) {
                    __hip_atomic_store(flags + ti * n_split + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(xcd_of + ti * n_split + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __hip_atomic_store(done + ti, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// The fold kernel: one workgroup of four waves per tile member (FoldShape,
// fold_body); the design is described at the top of fold_bf16.hip.
template <int R, int MAXB, int MODE>
__global__ __launch_bounds__(256) void fold_bf16_kernel(
    const uint16_t *__restrict__ dY, int64_t lddy, int T, int D, const uint16_t *__restrict__ P,
    int p_blocks, float *__restrict__ S, float *__restrict__ xbuf, int x_bytes, int *__restrict__ sync,
    int accumulate, int nblk, int n_tiles, int n_split, int steps_per, int spin_limit, int *__restrict__ timeouts) {
    __shared__ __attribute__((aligned(16))) char smem[FoldShape<R, MAXB>::LDS_BYTES];
    __shared__ int s_word;
    fold_body<R, MAXB, MODE>(smem, s_word, -1, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync, accumulate,
                             nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
}

}  // namespace logra
