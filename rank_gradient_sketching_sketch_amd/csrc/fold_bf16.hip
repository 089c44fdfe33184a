// Sketch stage 2 ("fold"): S (+)= dY^T P on the matrix cores, bf16 inputs,
// fp32 accumulation. P = c X Sigma^T is the projected microbatch that stage 1
// left in the workspace; S = G A^T with G = dY^T X is the sketch of the weight
// gradient ("NVIDIA's LoGRA fits RL post-training of a 27B model onto a single
// eight-GPU node", section "Why it matters").
//
// This is the dominant, HBM-bound kernel of the sketch: dY (T x d) is the big
// stream and every byte of it meets all r = 256 columns of P. What limits it
// on gfx950 is the bytes each compute unit pulls through its vector memory
// path: its own dY rows, plus all of P for the tokens it covers. Design:
//   * A tile is up to 10 blocks of 16 rows of S and all r columns; n_split
//     workgroups ("members") share a tile, each over one contiguous range of
//     the token steps. Splitting the tokens of taller tiles cuts the P bytes
//     per compute unit (for d = 18944: 128 tiles of 144-160 rows x 2 token
//     halves rather than 256 tiles of 64-80 rows x all tokens), and dY is
//     still read once. Kernel instances are built for tiles of at most 5 or
//     at most 10 blocks; the waves compute every block of the instance but the
//     last unconditionally (products past the tile are never stored), which
//     keeps the unrolled steps free of branches.
//   * dY is token-major, but the MFMA wants 8 consecutive tokens per lane. Each
//     thread streams 16-byte chunks of dY rows (8 columns of one token) into a
//     3-slot LDS ring, several steps of 32 tokens ahead in registers; the waves
//     then read operand fragments with the gfx950 transpose read
//     ds_read_b64_tr_b16 (one 4 x 16 block per 16-lane group, column j to lane
//     j). P is stored by stage 1 in operand-fragment order, so its fragments
//     come straight from L2 into registers. The four waves split the r columns
//     (64 each), so no P fragment is read twice in a workgroup.
//   * Barriers wait only for LDS traffic (workgroup fences on the local address
//     space), so the global prefetches stay in flight across them.
//   * Two members per tile add their partials without a second kernel: the
//     first finalizes the first half of the tile's row blocks, the second the
//     rest. Each writes its accumulators of the other's blocks to an exchange
//     buffer as raw MFMA fragments (1 KB per wave and block, device-coherent
//     stores), raises its flag, waits for the other's flag, and forms
//     S = [S +] (part_0 + part_1) for its rows; fp32 addition commutes, so the
//     result does not depend on which member finishes first. The flag is
//     raised with an agent-scope release (after a workgroup barrier, so it
//     covers every thread's fragment stores) and read with an agent-scope
//     acquire, which orders the fragments before it on any XCD.
//     Members take tickets from a counter when they start and a tile's two
//     members hold consecutive tickets (2i, 2i + 1). Tickets are drawn in
//     start order, so the workgroups that have started hold a prefix of the
//     tickets and at most one started member (the holder of the last, even
//     ticket) waits for a workgroup that has not started yet; that one starts
//     as soon as any slot on the chip frees up, and no two members wait on
//     each other in a cycle. Only two workgroups of a pair need ever be
//     resident together.
//     Workgroup ids are dealt round-robin over the 8 XCDs, so the ids of one
//     residue mod 8 draw tickets from a counter of their own and cover
//     consecutive tiles (the argument above then holds per counter): a pair
//     and its neighbouring tiles normally share one L2. Each member
//     publishes the XCD it runs on (hardware register XCC_ID); when both are
//     on one XCD the fragments go through that L2 with plain stores and
//     L1-bypassing loads, otherwise with device-coherent accesses.
//     Waits are bounded: a member that gives up writes its rows as NaN
//     rather than hanging, and counts itself in a caller-owned counter
//     (the fold_timeouts launch option). Stage 1 zeroes the counters, flags
//     and XCD words before each fold and the fold leaves them zero.
//   * More members per tile (small d, so that the grid still fills the chip)
//     each write their whole partial tile, and fold_reduce_kernel adds them in
//     member order.
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
template <int R, int MAXB>
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
    static constexpr int STAGE = R >= 256 ? 80 : 160;   // rows of the epilogue staging tile
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
// add); two, exchanging MFMA fragments within the kernel; or more, each
// writing its partial tile for fold_reduce_kernel to add.
enum FoldMode { kFoldSingle = 0, kFoldPair = 1, kFoldPartial = 2 };

template <int R, int MAXB, int MODE>
__global__ __launch_bounds__(256) void fold_bf16_kernel(
    const uint16_t *__restrict__ dY, int64_t lddy, int T, int D, const uint16_t *__restrict__ P,
    int p_blocks, float *__restrict__ S, float *__restrict__ xbuf, int x_bytes, int *__restrict__ sync,
    int accumulate, int nblk, int n_tiles, int n_split, int steps_per, int spin_limit, int *__restrict__ timeouts) {
    using Sh = FoldShape<R, MAXB>;
    constexpr int NBW = Sh::NBW, MBW = Sh::MBW, WM = Sh::WM, PF = Sh::PF, NCH = Sh::NCH;
    constexpr int kLdsRow = Sh::LDS_ROW;
    constexpr int kSlot = 32 * kLdsRow;                 // one step: 32 token rows
    constexpr int kTileLd = R + 4;                      // fp32 row stride of the staging tile in LDS
    constexpr int kRowChunks = R / 4;                   // 16-byte chunks per row of S
    constexpr int kStage = Sh::STAGE;
    constexpr int kOutChunks = (kStage * kRowChunks + 255) / 256;   // per thread per staged pass
    constexpr int kRingBytes = kFoldSlots * kSlot * 2;
    constexpr int kTileBytes = kStage * kTileLd * 4;
    // The dY ring during the loop, the staging tile in the epilogue.
    __shared__ __attribute__((aligned(16))) char smem[kRingBytes > kTileBytes ? kRingBytes : kTileBytes];
    __shared__ int s_word;
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
    if (MODE == kFoldPair) {
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
        own1 = MODE == kFoldSingle ? rows : 0;
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
    const __amdgpu_buffer_rsrc_t s_rs =
        __builtin_amdgcn_make_buffer_rsrc(S, 0, static_cast<int>(static_cast<int64_t>(D) * R * 4), 0x00020000);

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
    // read-modify-write S.
    for (int r0 = own0; r0 < own1; r0 += kStage) {
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
                old[c] = MODE == kFoldPair
                             ? old_pre[c]
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

// S = [S +] (part_0 + part_1 + ...): the members' partial tiles added in
// member order (small d, more than two members per tile).
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
    if (p.nblk >= 2 * kFoldWGs) {
        // tiles over two token halves when there are enough steps to split,
        // otherwise tiles over all tokens; at most 10 blocks a tile
        const int by_height = (p.nblk + 9) / 10;
        if (nsteps >= 8) {
            p.n_split = 2;
            p.n_tiles = by_height > kFoldWGs / 2 ? by_height : kFoldWGs / 2;
        } else {
            p.n_split = 1;
            p.n_tiles = by_height > kFoldWGs ? by_height : kFoldWGs;
        }
    } else {
        // small d: the tokens split so that the grid fills the compute units,
        // keeping the exchanged partials no larger than the dY they replace
        // and at least 4 steps per member; tiles of up to 10 blocks (longer
        // dY rows per step, less P per member) where they still make a
        // workgroup per compute unit, else tiles of 4 blocks
        const int64_t cap_bytes = T / (2 * R);
        auto splits = [&](int tiles) {
            int ns = kFoldWGs / tiles;
            if (ns > cap_bytes) ns = static_cast<int>(cap_bytes);
            if (ns > nsteps / 4) ns = nsteps / 4;
            if (ns > kFoldMaxSplit) ns = kFoldMaxSplit;
            return ns < 1 ? 1 : ns;
        };
        const int tall = (p.nblk + 9) / 10;
        if (tall * splits(tall) >= kFoldWGs) {
            p.n_tiles = tall;
        } else {
            p.n_tiles = (p.nblk + 3) / 4;
        }
        p.n_split = splits(p.n_tiles);
    }
    p.max_blocks = (p.nblk + p.n_tiles - 1) / p.n_tiles <= 5 ? 5 : 10;
    p.steps_per = (nsteps + p.n_split - 1) / p.n_split;
    p.n_split = (nsteps + p.steps_per - 1) / p.steps_per;
    const size_t align = 256;
    if (p.n_split == 2) {
        // fragments of every block of every tile, then the sync words
        p.xbuf_bytes = (static_cast<size_t>(p.n_tiles) * 2 * p.max_blocks * 16 * R * 4 + align - 1) / align * align;
        // ticket counter, one counter per id group, a flag and an XCD per
        // member, a done count per tile
        p.sync_words = 1 + kXcds + 2 * p.n_tiles * p.n_split + p.n_tiles;
        p.sync_bytes = (static_cast<size_t>(p.sync_words) * 4 + align - 1) / align * align;
    } else if (p.n_split > 2) {
        // one d x r partial per member
        p.xbuf_bytes = (static_cast<size_t>(p.n_split) * D * R * 4 + align - 1) / align * align;
    }
    return p;
}

template <int R>
static hipError_t fold_r(int64_t T, int64_t D, const uint16_t *dY, int64_t lddy, const uint16_t *P,
                         int p_blocks, float *S, int accumulate, void *scratch, const FoldWait &wait,
                         hipStream_t st) {
    const FoldPlan p = plan_fold_bf16(T, D, R);
    float *xbuf = static_cast<float *>(scratch);
    int *sync = reinterpret_cast<int *>(static_cast<char *>(scratch) + p.xbuf_bytes);
    auto kernel = fold_bf16_kernel<R, 5, kFoldSingle>;
    if (p.n_split > 2)
        kernel = p.max_blocks == 5 ? fold_bf16_kernel<R, 5, kFoldPartial> : fold_bf16_kernel<R, 10, kFoldPartial>;
    else if (p.n_split == 2)
        kernel = p.max_blocks == 5 ? fold_bf16_kernel<R, 5, kFoldPair> : fold_bf16_kernel<R, 10, kFoldPair>;
    else if (p.max_blocks == 10)
        kernel = fold_bf16_kernel<R, 10, kFoldSingle>;
    hipLaunchKernelGGL(kernel, dim3(p.n_tiles * p.n_split), dim3(256), 0, st, dY, lddy, static_cast<int>(T),
                       static_cast<int>(D), P, p_blocks, S, xbuf, static_cast<int>(p.xbuf_bytes), sync, accumulate,
                       p.nblk, p.n_tiles, p.n_split, p.steps_per, wait.spin_limit, wait.timeouts);
    if (p.n_split > 2) {
        const int64_t n = D * R;
        hipLaunchKernelGGL(fold_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, xbuf, p.n_split, n, S,
                           accumulate);
    }
    return hipGetLastError();
}

hipError_t launch_fold_bf16_tiles(int R, int64_t T, int64_t D, const uint16_t *dY, int64_t lddy,
                                  const uint16_t *P, int p_blocks, float *S, int accumulate,
                                  void *scratch, const FoldWait &wait, hipStream_t st) {
    switch (R) {
    case 32: return fold_r<32>(T, D, dY, lddy, P, p_blocks, S, accumulate, scratch, wait, st);
    case 64: return fold_r<64>(T, D, dY, lddy, P, p_blocks, S, accumulate, scratch, wait, st);
    case 128: return fold_r<128>(T, D, dY, lddy, P, p_blocks, S, accumulate, scratch, wait, st);
    case 256: return fold_r<256>(T, D, dY, lddy, P, p_blocks, S, accumulate, scratch, wait, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
