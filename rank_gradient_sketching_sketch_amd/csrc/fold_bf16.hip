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
//     still read once. Where the two halves would add their partials inside
//     the kernel, the split is taken only where all of P is more than 1 MB
//     per compute unit (T r > 2^19) or r = 256: below that the exchange and
//     its waits cost more than the halved P bytes save (at d = 18944 and
//     4096 tokens, r = 32: 48 -> 38 us per launch without the split; r = 256:
//     the split stays). Kernel instances are built for tiles of at most 5 or
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
//   * Split mode (logra_sketch_fold_parts) keeps the sketch of a step in n
//     parts while its microbatches arrive: member 0 of every tile adds its
//     partial to S, member q > 0 to part q - 1, each over the whole tile, so
//     members neither exchange nor wait; the step's last fold then adds the
//     parts into S in part order (fold_reduce_kernel).
//
// This file is compiled with the accumulators in vector registers rather
// than the accumulation registers (the build's per-file flag): the unrolled
// loop then keeps each accumulator where it is instead of rotating values
// between the two register files, which made the split- and single-mode
// folds about 3 % faster. The pair-mode instances run slower that way and
// are built in fold_pair_bf16.hip without it.
#include "fold_body.hpp"

namespace logra {

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

FoldPlan plan_fold_bf16(int64_t T, int64_t D, int R, bool parts) {
    FoldPlan p;
    if (T <= 0) return p;
    p.nblk = static_cast<int>((D + 15) / 16);
    const int nsteps = static_cast<int>((T + 31) / 32);
    if (p.nblk >= 2 * kFoldWGs) {
        // tiles over two token halves when there are enough steps to split
        // and halving each member's projection bytes pays for the split
        // (always with parts, which need no exchange; with the in-kernel
        // exchange only where all of P is more than 1 MB per compute unit,
        // T r > 2^19, or r = 256: below that the exchange and its waits cost
        // more than the projection bytes they save), otherwise tiles over all
        // tokens; at most 10 blocks a tile
        const int by_height = (p.nblk + 9) / 10;
        const bool split_pays = parts || R > 128 || T * static_cast<int64_t>(R) > (int64_t(1) << 19);
        if (nsteps >= 8 && split_pays) {
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
    if (p.n_split == 2)
        return launch_fold_pair_bf16(R, p.max_blocks, p.n_tiles * p.n_split, st, dY, lddy, static_cast<int>(T),
                                     static_cast<int>(D), P, p_blocks, S, xbuf, static_cast<int>(p.xbuf_bytes), sync,
                                     accumulate, p.nblk, p.n_tiles, p.n_split, p.steps_per, wait.spin_limit,
                                     wait.timeouts);
    auto kernel = fold_bf16_kernel<R, 5, kFoldSingle>;
    if (p.n_split > 2)
        kernel = p.max_blocks == 5 ? fold_bf16_kernel<R, 5, kFoldPartial> : fold_bf16_kernel<R, 10, kFoldPartial>;
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

template <int R>
static hipError_t fold_parts_r(int64_t T, int64_t D, const uint16_t *dY, int64_t lddy, const uint16_t *P,
                               int p_blocks, float *S, float *parts, int phase, hipStream_t st) {
    const FoldPlan p = plan_fold_bf16(T, D, R, true);
    const int first = phase & 1, last = phase & 2;
    auto kernel = fold_bf16_kernel<R, 5, kFoldSingle>;
    if (p.n_split > 1)
        kernel = p.max_blocks == 5 ? fold_bf16_kernel<R, 5, kFoldSplit> : fold_bf16_kernel<R, 10, kFoldSplit>;
    else if (p.max_blocks == 10)
        kernel = fold_bf16_kernel<R, 10, kFoldSingle>;
    hipLaunchKernelGGL(kernel, dim3(p.n_tiles * p.n_split), dim3(256), 0, st, dY, lddy, static_cast<int>(T),
                       static_cast<int>(D), P, p_blocks, S, parts, 0, nullptr, first ? 0 : 1, p.nblk, p.n_tiles,
                       p.n_split, p.steps_per, 0, nullptr);
    if (last && p.n_split > 1) {
        const int64_t n = D * R;
        hipLaunchKernelGGL(fold_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, parts, p.n_split - 1,
                           n, S, 1);
    }
    return hipGetLastError();
}

size_t fold_parts_bytes_bf16(int64_t T, int64_t D, int R) {
    const FoldPlan p = plan_fold_bf16(T, D, R, true);
    return p.n_split > 1 ? static_cast<size_t>(p.n_split - 1) * D * R * 4 : 0;
}

hipError_t launch_fold_parts_bf16(int R, int64_t T, int64_t D, const uint16_t *dY, int64_t lddy,
                                  const uint16_t *P, int p_blocks, float *S, float *parts, int phase,
                                  hipStream_t st) {
    switch (R) {
    case 32: return fold_parts_r<32>(T, D, dY, lddy, P, p_blocks, S, parts, phase, st);
    case 64: return fold_parts_r<64>(T, D, dY, lddy, P, p_blocks, S, parts, phase, st);
    case 128: return fold_parts_r<128>(T, D, dY, lddy, P, p_blocks, S, parts, phase, st);
    case 256: return fold_parts_r<256>(T, D, dY, lddy, P, p_blocks, S, parts, phase, st);
    default: return hipErrorInvalidValue;
    }
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
