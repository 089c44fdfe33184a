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
// contraction over d runs in chunks of 64: every thread moves 8 16-byte
// pieces of dY (256 tokens x 64) and 8 of W (64 x 256 columns) per chunk from
// HBM into registers two chunks ahead of use, then into one of two LDS
// buffers, so each wait is for a load issued two chunks earlier. dY rows
// (144 bytes with padding, so the 16 rows of a fragment read fall on
// different banks) give the A operand as 16-byte reads; W rows are read
// transposed with ds_read_b64_tr_b16, the B operand (8 consecutive d of one
// column per lane). Loads go through buffer views: tokens past T, rows past
// d and columns past k read as zero and are not written. The finished tile
// is rounded to bf16 (nearest even), staged in LDS and written as whole
// 16-byte pieces of dX rows. With one wave per SIMD the chunk's global
// loads, LDS reads and LDS writes are interleaved one by one with its MFMAs
// (scheduling barriers), which took the product at the 7B up shape from
// 690 to 564 us.
#include "fold_body.hpp"

namespace logra {

constexpr int kDxBM = 256, kDxBN = 256, kDxBK = 64;
constexpr int kDxARow = kDxBK + 8;            // bf16 per dY row in LDS (144 bytes)
constexpr int kDxBRow = kDxBN + 16;           // bf16 per W row in LDS (544 bytes)
constexpr int kDxABytes = kDxBM * kDxARow * 2;
constexpr int kDxBBytes = kDxBK * kDxBRow * 2;
constexpr int kDxLds = 2 * (kDxABytes + kDxBBytes);
constexpr int kDxCRow = kDxBN + 8;            // bf16 per row of the staged dX tile (528 bytes)
static_assert(kDxBM * kDxCRow * 2 <= kDxLds, "the dX tile is staged in the operand buffers");
constexpr int kDxFoldMaxB = 10;               // 16-row blocks per fold tile
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

__device__ __forceinline__ void dx_tile(char *smem, const DxArgs &a, int tm, int tn) {
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
    uint16_t *lds_a[2] = {reinterpret_cast<uint16_t *>(smem),
                          reinterpret_cast<uint16_t *>(smem + kDxABytes)};
    uint16_t *lds_b[2] = {reinterpret_cast<uint16_t *>(smem + 2 * kDxABytes),
                          reinterpret_cast<uint16_t *>(smem + 2 * kDxABytes + kDxBBytes)};

    // This thread's 8 pieces of dY (rows tid / 8 + 32 j, columns 8 (tid % 8)
    // .. +7 of the chunk) and 8 pieces of W (rows tid / 32 + 8 j, columns
    // 8 (tid % 32) .. +7), j = 0..7: a base per thread plus uniform strides.
    const int a_r0 = tid >> 3, a_c = 8 * (tid & 7);
    const int b_r0 = tid >> 5, b_c = 8 * (tid & 31);
    const uint32_t a_base = static_cast<uint32_t>((static_cast<int64_t>(t0 + a_r0) * a.lddy + a_c) * 2);
    const uint32_t a_jstep = static_cast<uint32_t>(a.lddy * 2 * 32);
    const uint32_t b_base = static_cast<uint32_t>((static_cast<int64_t>(b_r0) * a.ldw + n0 + b_c) * 2);
    const uint32_t b_jstep = static_cast<uint32_t>(a.ldw * 2 * 8);
    const uint32_t b_chunk_bytes = static_cast<uint32_t>(a.ldw * 2 * kDxBK);
    const int a_rows_left = a.T - t0 - a_r0;          // piece j is a token when 32 j < a_rows_left
    const bool b_col_ok = n0 + b_c < a.K;
    const int a_l0 = a_r0 * kDxARow + a_c, b_l0 = b_r0 * kDxBRow + b_c;
    auto load_chunk = [&](int c, u32x4_t (&ra)[8], u32x4_t (&rb)[8]) {
        const int d0 = c * kDxBK;
        const bool a_col_ok = d0 + a_c < a.D;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t ao = (a_col_ok && 32 * j < a_rows_left) ? a_base + 2u * d0 + j * a_jstep : kOob;
            ra[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rs, ao, 0, 0));
            const uint32_t bo = (b_col_ok && d0 + b_r0 + 8 * j < a.D)
                                    ? b_base + static_cast<uint32_t>(c) * b_chunk_bytes + j * b_jstep
                                    : kOob;
            rb[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rs, bo, 0, 0));
        }
    };
    auto store_chunk = [&](int buf, const u32x4_t (&ra)[8], const u32x4_t (&rb)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *reinterpret_cast<u32x4_t *>(lds_a[buf] + a_l0 + 32 * j * kDxARow) = ra[j];
            *reinterpret_cast<u32x4_t *>(lds_b[buf] + b_l0 + 8 * j * kDxBRow) = rb[j];
        }
    };

    f32x4_t acc[8][8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = zero_f32x4();

    auto compute = [&](int buf) {
        const uint16_t *A = lds_a[buf];
        const uint16_t *Bm = lds_b[buf];
#pragma unroll
        for (int ks = 0; ks < kDxBK / 32; ++ks) {
            u32x4_t af[8], bf[8];
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
                af[mb] = *reinterpret_cast<const u32x4_t *>(A + (128 * wm + 16 * mb + i16) * kDxARow + 32 * ks + 8 * g);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const uint16_t *p = Bm + (32 * ks + 8 * g + (i16 >> 2)) * kDxBRow + 128 * wn + 16 * nb + 4 * (i16 & 3);
                const u32x2_t lo = lds_read_tr(p);
                const u32x2_t hi = lds_read_tr(p + 4 * kDxBRow);
                bf[nb] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
            }
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_bf16(af[mb], bf[nb], acc[mb][nb]);
        }
    };

    // Register ring of two chunks: rg[c % 2] holds chunk c from its load
    // (two chunks ahead) until it is stored into LDS buffer c % 2 (one ahead).
    const int nck = (a.D + kDxBK - 1) / kDxBK;
    u32x4_t rga[2][8], rgb[2][8];
    load_chunk(0, rga[0], rgb[0]);
    if (nck > 1) load_chunk(1, rga[1], rgb[1]);
    store_chunk(0, rga[0], rgb[0]);
    lds_barrier();
    for (int c0 = 0; c0 < nck; c0 += 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = c0 + p;
            if (c < nck) {
                // Loads and stores are unconditional, so that the chunk is one
                // block of code the scheduler can interleave (past the last
                // chunk every offset is out of range and reads zero, and the
                // buffer stored then is never read). With one wave per SIMD
                // the matrix cores idle whenever the wave issues a run of
                // other instructions; one MFMA between each of the chunk's 16
                // global loads, 48 LDS reads and 16 LDS writes keeps them fed.
                load_chunk(c + 2, rga[p], rgb[p]);
                compute(p);
                store_chunk(p ^ 1, rga[p ^ 1], rgb[p ^ 1]);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
                }
#pragma unroll
                for (int i = 0; i < 48; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
                }
                lds_barrier();
            }
        }
    }

    // dX tile: rounded to bf16, staged row-major in LDS, written as 16-byte
    // pieces of rows. Lane (i16, g) of block (mb, nb) holds rows
    // 16 mb + 4 g + e, column 16 nb + i16 of its quarter.
    uint16_t *ct = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ct[(128 * wm + 16 * mb + 4 * g + e) * kDxCRow + 128 * wn + 16 * nb + i16] =
                    __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mb][nb][e]));
    lds_barrier();
#pragma unroll 4
    for (int j = 0; j < (kDxBM * kDxBN / 8) / 256; ++j) {
        const int q = tid + 256 * j;
        const int row = q >> 5, col = 8 * (q & 31);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ct + row * kDxCRow + col);
        const uint32_t off = (t0 + row < a.T && n0 + col < a.K)
                                 ? static_cast<uint32_t>((static_cast<int64_t>(t0 + row) * a.lddx + n0 + col) * 2)
                                 : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(v, c_rs, off, 0, 0);
    }
}

template <int R>
__global__ __launch_bounds__(256) void dx_sketch_kernel(DxArgs a) {
    constexpr int kFoldLds = FoldShape<R, kDxFoldMaxB>::LDS_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[kDxLds > kFoldLds ? kDxLds : kFoldLds];
    __shared__ int s_word;
    const int id = static_cast<int>(blockIdx.x);
    if (id < a.n_fold) {
        // the fold over tiles id, id + n_fold, ...: each over all tokens, as
        // the sketch kernel's single-member mode
        const int nsteps = (a.T + 31) / 32;
        for (int t = id; t < a.fold_tiles; t += a.n_fold) {
            fold_body<R, kDxFoldMaxB, kFoldSingle>(smem, s_word, t, a.dY, a.lddy, a.T, a.D, a.P, a.p_blocks, a.S,
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
    dx_tile(smem, a, tile / a.n_tn, tile % a.n_tn);
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
