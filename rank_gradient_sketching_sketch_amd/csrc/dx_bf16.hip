// Backward input gradient of a sketched projection, dX = dY W, in the same
// launch as the sketch's fold S (+)= dY^T P, bf16 inputs, fp32 accumulation.
//
// In the backward pass of a linear layer Y = X W^T (W is d x k, [out, in]),
// the input gradient is dX = dY W. The caller computes it anyway, from the
// same output gradient dY (T x d) that the sketch accumulates into S during
// backpropagation ("NVIDIA's LoGRA fits RL post-training of a 27B model onto
// a single eight-GPU node", section "Why it matters"). The two products are
// opposite kinds of work: dX is a large dense contraction (2 T d k FLOPs)
// bound by the matrix cores, the fold streams dY once and is bound by memory.
// A fold inside the product's tile loop would contract over the tokens of
// one tile only, leaving T / 256 partial sketches per row of S to be added
// across workgroups; instead this kernel runs the two side by side in one
// launch. The first workgroups run the fold over tiles of up to 10 blocks of
// 16 rows of S, all tokens each (no partial sums leave a workgroup; the fold
// body is the sketch kernel's own, fold_body.hpp), looping over the tiles;
// the rest compute 256 x 256 tiles of dX on the matrix cores. The fold uses
// the compute units and the memory bandwidth the product leaves free: at
// T = 4096, k = 3584 there are 224 product tiles for 256 compute units.
//
// Product tiles (v_mfma_f32_16x16x32_bf16). Four waves each own a 128 x 128
// quarter of the tile (8 x 8 accumulator blocks, 256 registers). The
// contraction over d runs in chunks of 32 through a ring of four LDS stages:
// buffer loads that write LDS directly fill chunk c + 4 while chunk c is
// multiplied, so each wait is for loads issued three chunks earlier, and the
// next chunk's operand fragments are read between the current chunk's
// MFMAs. dY rows give the A operand as 16-byte reads; W rows are read
// transposed with ds_read_b64_tr_b16, the B operand (8 consecutive d of one
// column per lane). Loads go through buffer views: tokens past T, rows past
// d and columns past k read as zero and are not written. The finished tile
// is rounded to bf16 (nearest even), staged in LDS and written as whole
// 16-byte pieces of dX rows.
#include "fold_body.hpp"

namespace logra {

constexpr int kDxBM = 256, kDxBN = 256, kDxBK = 32;
constexpr int kDxStages = 4;                  // LDS ring: chunk c in stage c % 4
constexpr int kDxAStage = kDxBM * kDxBK * 2;  // 256 token rows of 64 bytes
constexpr int kDxBStage = kDxBK * kDxBN * 2;  // 32 rows of d, 512 bytes each
constexpr int kDxStageBytes = kDxAStage + kDxBStage;
constexpr int kDxCRow = kDxBN + 8;            // bf16 per row of the staged dX tile (528 bytes)
constexpr int kDxCRowsPerStage = kDxBM / kDxStages;   // the dX tile is staged over the four stages
constexpr int kDxFoldMaxB = 10;               // 16-row blocks per fold tile
constexpr int kDxFoldStage = 32;              // rows per pass of the fold's epilogue (it has one stage of LDS)
constexpr int kDxStageLds = kDxStageBytes > kDxCRowsPerStage * kDxCRow * 2 ? kDxStageBytes
                                                                            : kDxCRowsPerStage * kDxCRow * 2;
static_assert(FoldShape<256, kDxFoldMaxB, kDxFoldStage>::LDS_BYTES <= kDxStageLds, "the fold fits one stage");
constexpr int kDxChipWGs = 256;               // one workgroup per compute unit
constexpr int kDxFoldWGs = 32;                // fold workgroups beside a full grid of product tiles

struct DxArgs {
    const uint16_t *dY;
    int64_t lddy;
    const uint16_t *W;
    int64_t ldw;
    uint16_t *dX;
    int64_t lddx;
    int T, D, K;
    int n_tm, n_tn;        // product tiles (tokens x columns of k)
    int n_fold;            // fold workgroups (ids 0 .. n_fold - 1); 0: the product only
    const uint16_t *P;     // the projection (fold operand layout), p_blocks blocks of 32 tokens
    int p_blocks;
    float *S;
    int accumulate;
    int fold_nblk, fold_tiles;
    int spin_limit;
    int *timeouts;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Swizzled stage layouts. The loads write LDS straight from memory, 1 KB per
// wave instruction in lane order, so rows cannot be padded; instead the
// 16-byte granules of a row are permuted, and each lane fetches the granule
// that belongs at its position. A: token row t (4 granules of 8 d) keeps
// granule q at q ^ ((t >> 2) & 3), so the 16 rows of a fragment read fall
// on 16 different 16-byte bank groups. B: row j of d (32 granules of 8
// columns) keeps granule q at q ^ dx_bsw(j), so the 8 rows that 32 lanes of
// a transposed read touch (4 rows each of two 8-row groups) fall on 16
// different bank groups for each pair of granules.
__device__ __forceinline__ int dx_bsw(int j) { return ((j & 3) << 1) | (((j >> 3) & 1) << 3); }

// The four stages are separate LDS arrays, so that the compiler can tell
// the fragment reads of one stage from the loads still landing in the
// others (with one array it waits for every load before each read).
__device__ __forceinline__ void dx_tile(char *s0, char *s1, char *s2, char *s3, const DxArgs &a, int tm, int tn) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int i16 = lane & 15, g = lane >> 4;
    const int t0 = tm * kDxBM, n0 = tn * kDxBN;
    constexpr uint32_t kOob = 0x80000000u;
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.dY), 0, static_cast<int>(static_cast<int64_t>(a.T) * a.lddy * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.W), 0, static_cast<int>(static_cast<int64_t>(a.D) * a.ldw * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t c_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.dX, 0, static_cast<int>(static_cast<int64_t>(a.T) * a.lddx * 2), 0x00020000);

    // The chunk's loads: wave w's instruction i fills 1 KB block 4 w + i of
    // each operand's stage. A block: token rows 16 (4 w + i) .. +15, lane L
    // at row 16 (4 w + i) + L / 4, position L % 4. B block: rows of d
    // 2 (4 w + i) and +1, lane L at row 2 (4 w + i) + L / 32, position
    // L % 32. A base offset per instruction plus a uniform step per chunk.
    uint32_t a_off[4], b_off[4];
    int a_q[4], b_row[4];
    bool a_ok[4], b_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int blk = 4 * wave + i;
        const int ta = 16 * blk + (lane >> 2);
        a_q[i] = (lane & 3) ^ ((ta >> 2) & 3);
        a_ok[i] = t0 + ta < a.T;
        a_off[i] = a_ok[i] ? static_cast<uint32_t>((static_cast<int64_t>(t0 + ta) * a.lddy + 8 * a_q[i]) * 2) : kOob;
        const int jb = 2 * blk + (lane >> 5);
        const int qb = (lane & 31) ^ dx_bsw(jb);
        b_row[i] = jb;
        b_ok[i] = n0 + 8 * qb < a.K;
        b_off[i] = b_ok[i] ? static_cast<uint32_t>((static_cast<int64_t>(jb) * a.ldw + n0 + 8 * qb) * 2) : kOob;
    }
    const uint32_t b_chunk_bytes = static_cast<uint32_t>(a.ldw * 2 * kDxBK);
    const int nck = (a.D + kDxBK - 1) / kDxBK;
    // chunk c into stage S (c % 4); past the last chunk every offset is out
    // of range and the stage is filled with zeros that are never read
    // The chunk's step is the uniform (scalar) offset of the loads; a lane
    // outside the operands takes the out-of-range offset, which no scalar
    // offset brings back in range.
    auto issue = [&](int c, auto stage_c) {
        constexpr int S = decltype(stage_c)::value;
        char *st = S == 0 ? s0 : S == 1 ? s1 : S == 2 ? s2 : s3;
        const int d0 = c * kDxBK;
        const int d_left = a.D - d0;   // <= 0 past the last chunk
        // (no step past the last chunk: every lane is out of range there,
        // and a step beyond the view must not wrap an offset back into it)
        const int a_step = d_left > 0 ? 2 * d0 : 0;
        const int b_step = d_left > 0 ? static_cast<int>(static_cast<uint32_t>(c) * b_chunk_bytes) : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ao = 8 * a_q[i] < d_left ? a_off[i] : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_void_t *)(st + (4 * wave + i) * 1024), 16, ao, a_step,
                                                     0, 0);
            const uint32_t bo = b_row[i] < d_left ? b_off[i] : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs, (lds_void_t *)(st + kDxAStage + (4 * wave + i) * 1024), 16,
                                                     bo, b_step, 0, 0);
        }
    };

    // Operand fragments of one chunk (v_mfma_f32_16x16x32_bf16): A, row
    // 128 wm + 16 mb + i16, d 8 g .. +7 (16 bytes); B, transposed reads of
    // rows 8 g .. +7 of d, column 128 wn + 16 nb + i16.
    auto read_frags = [&](auto stage_c, u32x4_t (&af)[8], u32x4_t (&bf)[8]) {
        constexpr int S = decltype(stage_c)::value;
        const char *A = S == 0 ? s0 : S == 1 ? s1 : S == 2 ? s2 : s3;
        const char *Bm = A + kDxAStage;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int t = 128 * wm + 16 * mb + i16;
            af[mb] = *reinterpret_cast<const u32x4_t *>(A + t * 64 + ((g ^ ((t >> 2) & 3)) << 4));
        }
        const int j_lo = 8 * g + (i16 >> 2), j_hi = j_lo + 4;
        const int sub = (i16 & 1) * 8;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int q = 16 * wn + 2 * nb + ((i16 & 3) >> 1);
            const u32x2_t lo = lds_read_tr(reinterpret_cast<const uint16_t *>(Bm + j_lo * 512 + ((q ^ dx_bsw(j_lo)) << 4) + sub));
            const u32x2_t hi = lds_read_tr(reinterpret_cast<const uint16_t *>(Bm + j_hi * 512 + ((q ^ dx_bsw(j_hi)) << 4) + sub));
            bf[nb] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
    };

    f32x4_t acc[8][8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = zero_f32x4();

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // Pipeline: chunks 0..3 in flight, then per chunk c: wait until chunk
    // c + 1 has landed (c + 2 and c + 3 may still be in flight) and the
    // fragment reads of chunk c are done; a barrier, after which every wave
    // has both (so stage c % 4 is free); the load of chunk c + 4 into it;
    // then chunk c's 64 MFMAs with chunk c + 1's 24 fragment reads between
    // them. Each wait is for loads issued three chunks earlier.
    u32x4_t af[2][8], bfr[2][8];
    issue(0, I0{});
    issue(1, I1{});
    issue(2, I2{});
    issue(3, I3{});
    __builtin_amdgcn_s_waitcnt(0x4078);   // vmcnt(24) expcnt(7) lgkmcnt(0): chunk 0 has landed
    __builtin_amdgcn_s_barrier();
    read_frags(I0{}, af[0], bfr[0]);
    auto step = [&](int c, auto stage_c) {
        constexpr int S = decltype(stage_c)::value;
        constexpr int F = S & 1;
        // vmcnt(16) expcnt(7) lgkmcnt(0): chunk c + 1 has landed, chunk c's
        // fragments are in registers
        __builtin_amdgcn_s_waitcnt(0x4070);
        __builtin_amdgcn_s_barrier();
        issue(c + 4, stage_c);
        read_frags(std::integral_constant<int, (S + 1) & 3>{}, af[F ^ 1], bfr[F ^ 1]);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_bf16(af[F][mb], bfr[F][nb], acc[mb][nb]);
        // one MFMA between each of the 8 loads and 24 fragment reads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // load
        }
#pragma unroll
        for (int i = 0; i < 24; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
    };
    for (int c0 = 0; c0 < nck; c0 += 4) {
        step(c0, I0{});
        if (c0 + 1 < nck) step(c0 + 1, I1{});
        if (c0 + 2 < nck) step(c0 + 2, I2{});
        if (c0 + 3 < nck) step(c0 + 3, I3{});
    }

    // dX tile: rounded to bf16, staged row-major in LDS, written as 16-byte
    // pieces of rows. Lane (i16, g) of block (mb, nb) holds rows
    // 16 mb + 4 g + e, column 16 nb + i16 of its quarter. The ring's last
    // loads (zeros past the last chunk) land before the staging overwrites it.
    // Tile rows 64 s .. 64 s + 63 go to stage s.
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    uint16_t *const ct[4] = {reinterpret_cast<uint16_t *>(s0), reinterpret_cast<uint16_t *>(s1),
                             reinterpret_cast<uint16_t *>(s2), reinterpret_cast<uint16_t *>(s3)};
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        uint16_t *cs = ct[2 * wm + mb / 4];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cs[(16 * (mb % 4) + 4 * g + e) * kDxCRow + 128 * wn + 16 * nb + i16] =
                    __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mb][nb][e]));
    }
    lds_barrier();
#pragma unroll 4
    for (int j = 0; j < (kDxBM * kDxBN / 8) / 256; ++j) {
        const int q = tid + 256 * j;
        const int row = q >> 5, col = 8 * (q & 31);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ct[row / kDxCRowsPerStage] +
                                                             (row % kDxCRowsPerStage) * kDxCRow + col);
        const uint32_t off = (t0 + row < a.T && n0 + col < a.K)
                                 ? static_cast<uint32_t>((static_cast<int64_t>(t0 + row) * a.lddx + n0 + col) * 2)
                                 : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(v, c_rs, off, 0, 0);
    }
}

template <int R>
__global__ __launch_bounds__(256) void dx_sketch_kernel(DxArgs a) {
    static_assert(FoldShape<R, kDxFoldMaxB, kDxFoldStage>::LDS_BYTES <= kDxStageLds, "the fold fits one stage");
    __shared__ __attribute__((aligned(16))) char s0[kDxStageLds];
    __shared__ __attribute__((aligned(16))) char s1[kDxStageLds];
    __shared__ __attribute__((aligned(16))) char s2[kDxStageLds];
    __shared__ __attribute__((aligned(16))) char s3[kDxStageLds];
    __shared__ int s_word;
    const int id = static_cast<int>(blockIdx.x);
    if (id < a.n_fold) {
        // the fold over tiles id, id + n_fold, ...: each over all tokens, as
        // the sketch kernel's single-member mode
        const int nsteps = (a.T + 31) / 32;
        for (int t = id; t < a.fold_tiles; t += a.n_fold) {
            fold_body<R, kDxFoldMaxB, kFoldSingle, kDxFoldStage>(s0, s_word, t, a.dY, a.lddy, a.T, a.D, a.P,
                                                                 a.p_blocks, a.S,
                                                   nullptr, 0, nullptr, a.accumulate, a.fold_nblk, a.fold_tiles,
                                                   1, nsteps, a.spin_limit, a.timeouts);
            __syncthreads();   // the next tile's ring reuses the LDS
        }
        return;
    }
    // product tiles: the workgroup ids of one XCD (id mod 8) take a
    // contiguous run of tiles in row-major (tm, tn) order, so they share
    // rows of dY in that XCD's L2
    const int gid = id - a.n_fold;
    const int G = a.n_tm * a.n_tn;
    const int tile = (G % kXcds == 0) ? (gid % kXcds) * (G / kXcds) + gid / kXcds : gid;
    dx_tile(s0, s1, s2, s3, a, tile / a.n_tn, tile % a.n_tn);
}

DxPlan plan_dx_bf16(int64_t T, int64_t D, int64_t K, int sketch) {
    DxPlan p;
    p.n_tm = static_cast<int>((T + kDxBM - 1) / kDxBM);
    p.n_tn = static_cast<int>((K + kDxBN - 1) / kDxBN);
    p.fold_nblk = static_cast<int>((D + 15) / 16);
    p.fold_tiles = (p.fold_nblk + kDxFoldMaxB - 1) / kDxFoldMaxB;
    p.n_fold = 0;
    if (sketch && T > 0) {
        // the compute units a grid of product tiles leaves free, at least
        // kDxFoldWGs, at most one per fold tile
        const int G = p.n_tm * p.n_tn;
        int spare = G % kDxChipWGs == 0 ? 0 : kDxChipWGs - G % kDxChipWGs;
        if (spare < kDxFoldWGs) spare = kDxFoldWGs;
        p.n_fold = spare < p.fold_tiles ? spare : p.fold_tiles;
    }
    return p;
}

// Whether the fold fits in the product's shadow: a fold workgroup streams
// all tokens of its tiles (rows of dY plus the whole projection, at about the
// 60 GB/s one compute unit pulls), and the product runs at about 700 TFLOP/s
// (both measured at the 7B shapes). Where the fold workgroups' share would
// outlast three quarters of the product (small d, so few fold tiles for all
// tokens), the product and the sketch kernel run one after the other instead.
bool dx_fuse_pays(int64_t T, int64_t D, int64_t K, int R) {
    const DxPlan p = plan_dx_bf16(T, D, K, 1);
    if (p.n_fold == 0) return false;
    const double tile_bytes = 2.0 * T * (16.0 * kDxFoldMaxB + R);
    const double per_wg = ((p.fold_tiles + p.n_fold - 1) / p.n_fold) * tile_bytes / 60e9;
    const double product = 2.0 * T * D * K / 700e12;
    return per_wg <= 0.75 * product;
}

template <int R>
static hipError_t dx_r(const DxArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(dx_sketch_kernel<R>, dim3(a.n_fold + a.n_tm * a.n_tn), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dx_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                          const uint16_t *W, int64_t ldw, uint16_t *dX, int64_t lddx, const uint16_t *P,
                          int p_blocks, float *S, int accumulate, int sketch, const FoldWait &wait,
                          hipStream_t st) {
    const DxPlan p = plan_dx_bf16(T, D, K, sketch);
    DxArgs a;
    a.dY = dY;
    a.lddy = lddy;
    a.W = W;
    a.ldw = ldw;
    a.dX = dX;
    a.lddx = lddx;
    a.T = static_cast<int>(T);
    a.D = static_cast<int>(D);
    a.K = static_cast<int>(K);
    a.n_tm = p.n_tm;
    a.n_tn = p.n_tn;
    a.n_fold = p.n_fold;
    a.P = P;
    a.p_blocks = p_blocks;
    a.S = S;
    a.accumulate = accumulate;
    a.fold_nblk = p.fold_nblk;
    a.fold_tiles = p.fold_tiles;
    a.spin_limit = wait.spin_limit;
    a.timeouts = wait.timeouts;
    if (a.n_tm * a.n_tn + a.n_fold == 0) return hipSuccess;
    switch (R) {
    case 32: return dx_r<32>(a, st);
    case 64: return dx_r<64>(a, st);
    case 128: return dx_r<128>(a, st);
    case 256: return dx_r<256>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
