// Apply pass 1 for bf16 compute: the per-row sums of squares of Ghat = S A
// and the step controller's reduction, from the r x r Gram matrix of the
// signs instead of a d x k reconstruction.
//
// RowAdam keeps one second moment per row ("NVIDIA's LoGRA fits RL
// post-training of a 27B model onto a single eight-GPU node", sections "What
// happened" and "Why it matters"); pass 1 needs rowsq_i = sum_j Ghat_ij^2 for
// it and the controller needs sum_i rowsq_i / (sqrt(v'_i) + eps)^2 ("LoGRA:
// Scaling LLM Reinforcement Learning...", paragraph "Step control."). With
// A = c Sigma,
//     rowsq_i = ||S_i A||^2 = c^2 S_i (Sigma Sigma^T) S_i^T = c^2 S_i M S_i^T,
// the same number up to rounding, for 2 r^2 (d + k) operations instead of
// 2 d k r. M_lm = k - 2 popcount(sigma_l xor sigma_m) is an exact integer
// (column tail masked). The diagonal part k ||S_i||^2 is summed in fp32; the
// off-diagonal part Y = S M_off runs on bf16 MFMA (S rounded to bf16 as in
// pass 2; M_off rounded to bf16, exact for |M_lm| <= 256) and is dotted with
// the fp32 S row.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

// M_off[l][m] (bf16, zero diagonal) = k - 2 popcount(sigma_l xor sigma_m),
// stored in MFMA operand order: the fragment of 16-row block lb and 32-wide
// step s of m is 1 KB, lane (n, g) holding M_off[16 lb + n][32 s + 8 g .. +7]
// in 16 bytes, so a wave loads one fragment as one contiguous kilobyte. A
// workgroup owns a 16 x 16 tile of (l, m); the sign words of its 32 rows are
// hashed into LDS 64 blocks at a time (rows padded by one word so the 16 rows
// of a column read fall on different banks) and each thread counts the sign
// differences of its pair.
constexpr int kGramChunk = 64;   // 64-bit words per row per chunk

__device__ __forceinline__ void gram_body(uint64_t key, int R, int K, uint16_t *__restrict__ M,
                                          uint64_t *__restrict__ slots, int n_slots, int bx, int by) {
    __shared__ uint64_t wl[16][kGramChunk + 1];
    __shared__ uint64_t wm[16][kGramChunk + 1];
    const int tid = threadIdx.x;
    // the rowsq kernel that follows finds its workgroups' partials by the
    // mark each one sets in its slot (and leaves the slots zero again)
    if (bx == 0 && by == 0)
        for (int i = tid; i < n_slots; i += 256) slots[i] = 0;
    const int l0 = by * 16, m0 = bx * 16;
    const int tl = tid >> 4, tm = tid & 15;
    const int nb = (K + 63) / 64;
    const int tail = K - 64 * (nb - 1);
    const uint64_t last_mask = tail == 64 ? ~0ull : ((1ull << tail) - 1ull);
    int pc = 0;
    for (int b0 = 0; b0 < nb; b0 += kGramChunk) {
        const int bn = min(kGramChunk, nb - b0);
        for (int idx = tid; idx < 2 * 16 * kGramChunk; idx += 256) {
            const int which = idx / (16 * kGramChunk);
            const int rem = idx - which * 16 * kGramChunk;
            const int row = rem / kGramChunk, bb = rem - row * kGramChunk;
            uint64_t w = 0;
            if (bb < bn) {
                w = sign_word(key, static_cast<uint32_t>((which ? m0 : l0) + row), static_cast<uint32_t>(b0 + bb));
                if (b0 + bb == nb - 1) w &= last_mask;   // columns past k do not count
            }
            (which ? wm : wl)[row][bb] = w;
        }
        __syncthreads();
        for (int bb = 0; bb < bn; ++bb) pc += __popcll(wl[tl][bb] ^ wm[tm][bb]);
        __syncthreads();
    }
    const int l = l0 + tl, m = m0 + tm;
    const float v = l == m ? 0.f : static_cast<float>(K - 2 * pc);
    const int frag = (l >> 4) * (R / 32) + (m >> 5);
    const int ln = (((m & 31) >> 3) << 4) | (l & 15);   // lane (n = l % 16, g = (m % 32) / 8)
    M[(static_cast<size_t>(frag) * 64 + ln) * 8 + (m & 7)] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

__global__ __launch_bounds__(256) void gram_kernel(uint64_t key, int R, int K, uint16_t *__restrict__ M,
                                                   uint64_t *__restrict__ slots, int n_slots) {
    gram_body(key, R, K, M, slots, n_slots, blockIdx.x, blockIdx.y);
}

// rowsq_i = c^2 (k ||S_i||^2 + sum_m S_im Y_im), Y^T = M_off S^T. A workgroup
// owns bpw blocks of 16 rows of S (the plan makes about one workgroup per
// compute unit) and stages them in LDS as fp32 (rows padded by 16 bytes, so
// the 16 rows of a fragment fall on different banks). Each of the four waves
// owns a quarter of the 16-row blocks of m and keeps their M_off fragments
// (the MFMA A operand, straight from L2) in registers for the whole
// workgroup, so M_off crosses each compute unit's memory path once and no
// LDS copy of it is needed. Per row block the waves build the bf16 S^T
// fragments (B operand) from LDS, form their 16 x 16 blocks of Y^T, and dot
// each with the fp32 S entries of the same (i, m), also accumulating the
// squares of those entries: every wave thus covers its m range of both sums,
// and the four waves' partials are added per row in wave order. The
// controller's sum ends in the same kernel: each workgroup publishes its
// partial as one 64-bit agent-scope atomic store of (mark << 32 | bits) into
// its own slot and is done. Workgroup 0 (dispatched first) then reads every
// slot with 64-bit atomic loads, polling each until its mark is set (a slot
// is a single atomic location, so a marked value is that workgroup's partial
// of this launch: no ordering between different locations is relied on),
// adds the partials in index order (fixed, so the result does not depend on
// the order the workgroups finish in), and clears the slots for the next
// call. No workgroup waits for an atomic's reply before it ends, and only
// workgroup 0 waits at all, which needs nothing of the others but that
// they run (it holds one compute unit while they do). The poll is bounded;
// if it gives up, sqnorm is NaN.
constexpr int kRowsqMaxBlocks = 8;   // 16-row blocks of S per workgroup (most)
constexpr int kRowsqWGs = 256;       // target workgroups (one per compute unit)
constexpr uint64_t kSlotMark = 1ull << 32;
constexpr int kSlotSpinLimit = 1 << 22;   // polls of one slot before the sum gives up

template <int R>
__device__ __forceinline__ void rowsq_body(const float *__restrict__ S, int D, int K,
                                           const uint16_t *__restrict__ M, float c,
                                           const float *__restrict__ v, float beta2, float eps,
                                           float *__restrict__ v_new, float *__restrict__ rowsq,
                                           uint64_t *__restrict__ slots, int bpw, float *__restrict__ sqnorm,
                                           int blk, int nblk) {
    constexpr int KS = R / 32;                    // 32-wide steps of the rank
    constexpr int NB = R / 16;                    // 16-row blocks of m
    constexpr int MPW = NB >= 4 ? NB / 4 : 1;     // blocks of m per wave
    constexpr int LD = R + 4;                     // fp32 stride of an S row in LDS
    constexpr int CPR = R / 4;                    // 16-byte chunks per S row
    constexpr int kMaxRows = kRowsqMaxBlocks * 16;
    constexpr int kChunks = (kMaxRows * CPR + 255) / 256;   // staging chunks per thread (most)
    __shared__ __attribute__((aligned(16))) float srow[kMaxRows * LD];
    __shared__ float2 part[4][kMaxRows];          // per wave and row: (dot, squares)
    __shared__ float terms[4];
    __shared__ float red[256];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int r0 = blk * bpw * 16;
    const int rows = min(bpw * 16, D - r0);
    const int mb0 = wave * MPW;
    const bool active = mb0 < NB;                 // r = 32: two of the four waves have no m block

    // 1. this wave's M_off fragments: row m = 16 (mb0 + j) + n, k = 32 s + 8 g .. +7
    // (fragment order: one contiguous kilobyte per fragment)
    u32x4_t mf[MPW][KS];
#pragma unroll
    for (int j = 0; j < MPW; ++j)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            mf[j][s] = active ? load_u32x4(M + (static_cast<size_t>((mb0 + j) * KS + s) * 64 + lane) * 8)
                              : zero_u32x4();
    // 2. the workgroup's S rows into LDS, every load in flight before the stores (rows past d as zero)
    {
        f32x4_t st[kChunks];
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = tid + 256 * q, row = idx / CPR, ch = idx - row * CPR;
            st[q] = row < rows ? *reinterpret_cast<const f32x4_t *>(S + static_cast<int64_t>(r0 + row) * R + 4 * ch)
                               : zero_f32x4();
        }
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = tid + 256 * q, row = idx / CPR, ch = idx - row * CPR;
            if (row < bpw * 16) *reinterpret_cast<f32x4_t *>(&srow[row * LD + 4 * ch]) = st[q];
        }
    }
    __syncthreads();

    // 3. per row block: this wave's blocks of Y^T (lane (n, g) gets
    // Y[i = 16 rb + n][m = 16 mb + 4 g + e]) dotted with S[i][m]
    for (int rb = 0; rb < bpw; ++rb) {
        const float *si = &srow[(16 * rb + n) * LD];
        float yd = 0.f, sq = 0.f;
        if (active) {
            u32x4_t sb[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(si + 32 * s + 8 * g);
                const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(si + 32 * s + 8 * g + 4);
                sb[s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                                pack_bf16x2(hi.z, hi.w)};
            }
#pragma unroll
            for (int j = 0; j < MPW; ++j) {
                f32x4_t acc = zero_f32x4();
#pragma unroll
                for (int s = 0; s < KS; ++s) acc = mfma_bf16(mf[j][s], sb[s], acc);
                const f32x4_t sv = *reinterpret_cast<const f32x4_t *>(si + 16 * (mb0 + j) + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    yd = fmaf(sv[e], acc[e], yd);
                    sq = fmaf(sv[e], sv[e], sq);
                }
            }
        }
        // the four lanes of a row (g = 0..3), fixed butterfly order
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            yd += __shfl_xor(yd, off, 64);
            sq += __shfl_xor(sq, off, 64);
        }
        if (g == 0) part[wave][16 * rb + n] = make_float2(yd, sq);
    }
    __syncthreads();

    // 4. rowsq, v' (both stored) and the controller's term, one thread per row
    float term = 0.f;
    if (tid < rows) {
        const float2 p0 = part[0][tid], p1 = part[1][tid], p2 = part[2][tid], p3 = part[3][tid];
        const float yd = ((p0.x + p1.x) + p2.x) + p3.x;
        const float sq = ((p0.y + p1.y) + p2.y) + p3.y;
        const int i = r0 + tid;
        const float rq = (c * c) * fmaf(static_cast<float>(K), sq, yd);
        if (rowsq) rowsq[i] = rq;
        const float vn = beta2 * v[i] + (1.f - beta2) * (rq / static_cast<float>(K));
        v_new[i] = vn;
        const float u = 1.f / (sqrtf(vn) + eps);
        term = rq * u * u;
    }
    // per-workgroup partial of the controller's reduction, fixed order
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) term += __shfl_xor(term, off, 64);
    if (lane == 0) terms[wave] = term;
    __syncthreads();
    if (tid == 0) {
        const float pw = ((terms[0] + terms[1]) + terms[2]) + terms[3];
        __hip_atomic_store(slots + blk, kSlotMark | __float_as_uint(pw), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blk != 0) return;
    // sqnorm = the partials added in a fixed order: strided per thread, then a tree
    float t = 0.f;
    bool ok = true;
    for (int i = tid; i < nblk; i += 256) {
        uint64_t w = __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spins = 0; !(w & kSlotMark) && spins < kSlotSpinLimit; ++spins) {
            __builtin_amdgcn_s_sleep(1);
            w = __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ok = ok && (w & kSlotMark);
        t += __uint_as_float(static_cast<uint32_t>(w));
        __hip_atomic_store(slots + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    red[tid] = ok ? t : __builtin_nanf("");
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) sqnorm[0] = red[0];
}

template <int R>
__global__ __launch_bounds__(256) void rowsq_gram_kernel(const float *__restrict__ S, int D, int K,
                                                         const uint16_t *__restrict__ M, float c,
                                                         const float *__restrict__ v, float beta2,
                                                         float eps, float *__restrict__ v_new,
                                                         float *__restrict__ rowsq,
                                                         uint64_t *__restrict__ slots, int bpw,
                                                         float *__restrict__ sqnorm) {
    rowsq_body<R>(S, D, K, M, c, v, beta2, eps, v_new, rowsq, slots, bpw, sqnorm, blockIdx.x,
                  gridDim.x);
}

// Pass 1 of several matrices of one rank in two launches: the Gram matrices
// of all of them (grid z = matrix), then every matrix's row blocks in one
// grid, each workgroup finding its matrix from the running block counts.
// Each matrix keeps its own workspace slice and sqnorm, and the
// per-matrix arithmetic is the single-matrix kernels' own, so the results
// are bit-identical to calling them one matrix at a time.
template <int R>
__global__ __launch_bounds__(256) void gram_batch_kernel(SqnormBatch b) {
    const SqnormItem &it = b.item[blockIdx.z];
    gram_body(it.key, R, it.K, it.M, it.slots, it.n_wg, blockIdx.x, blockIdx.y);
}

template <int R>
__global__ __launch_bounds__(256) void rowsq_batch_kernel(SqnormBatch b) {
    int j = 0;
    while (j + 1 < b.n && static_cast<int>(blockIdx.x) >= b.item[j + 1].wg_begin) ++j;
    const SqnormItem &it = b.item[j];
    rowsq_body<R>(it.S, it.D, it.K, it.M, it.c, it.v, b.beta2, b.eps, it.v_new, it.rowsq, it.slots, it.bpw,
                  b.sqnorm + j, static_cast<int>(blockIdx.x) - it.wg_begin, it.n_wg);
}

SqnormPlan plan_sqnorm_bf16(int64_t D, int64_t K, int R) {
    SqnormPlan p;
    (void)K;
    (void)R;
    const int64_t nblk = (D + 15) / 16;
    int64_t bpw = (nblk + kRowsqWGs - 1) / kRowsqWGs;
    if (bpw > kRowsqMaxBlocks) bpw = kRowsqMaxBlocks;
    if (bpw < 1) bpw = 1;
    p.rows_per_block = static_cast<int>(16 * bpw);
    p.n_blocks = static_cast<int>((D + p.rows_per_block - 1) / p.rows_per_block);
    const size_t align = 256;
    p.partial_bytes = (static_cast<size_t>(p.n_blocks) * 8 + align - 1) / align * align;
    p.gram_bytes = (static_cast<size_t>(R) * R * 2 + align - 1) / align * align;
    return p;
}

template <int R>
static hipError_t sqnorm_r(const ApplyArgs &a, void *ws, int parts, hipStream_t st) {
    const SqnormPlan p = plan_sqnorm_bf16(a.D, a.K, R);
    char *base = static_cast<char *>(ws);
    uint64_t *slots = reinterpret_cast<uint64_t *>(base);
    uint16_t *M = reinterpret_cast<uint16_t *>(base + p.partial_bytes);
    const int K = static_cast<int>(a.K);
    if (parts & kSqnormGram)
        hipLaunchKernelGGL(gram_kernel, dim3(R / 16, R / 16), dim3(256), 0, st, a.key, R, K, M, slots,
                           p.n_blocks);
    if (parts & kSqnormRows)
        hipLaunchKernelGGL(rowsq_gram_kernel<R>, dim3(p.n_blocks), dim3(256), 0, st, a.S,
                           static_cast<int>(a.D), K, M, a.c, a.v_in, a.beta2, a.eps, a.v_new_out, a.rowsq_out,
                           slots, p.rows_per_block / 16, a.sqnorm);
    return hipGetLastError();
}

template <int R>
static hipError_t sqnorm_batch_r(const SqnormBatch &b, hipStream_t st) {
    int total = 0;
    for (int j = 0; j < b.n; ++j) total += b.item[j].n_wg;
    hipLaunchKernelGGL(gram_batch_kernel<R>, dim3(R / 16, R / 16, b.n), dim3(256), 0, st, b);
    hipLaunchKernelGGL(rowsq_batch_kernel<R>, dim3(total), dim3(256), 0, st, b);
    return hipGetLastError();
}

hipError_t launch_sqnorm_batch_bf16(int R, const SqnormBatch &b, hipStream_t st) {
    switch (R) {
    case 32: return sqnorm_batch_r<32>(b, st);
    case 64: return sqnorm_batch_r<64>(b, st);
    case 128: return sqnorm_batch_r<128>(b, st);
    case 256: return sqnorm_batch_r<256>(b, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sqnorm_bf16(const ApplyArgs &a, void *ws, hipStream_t st, int parts) {
    switch (a.R) {
    case 32: return sqnorm_r<32>(a, ws, parts, st);
    case 64: return sqnorm_r<64>(a, ws, parts, st);
    case 128: return sqnorm_r<128>(a, ws, parts, st);
    case 256: return sqnorm_r<256>(a, ws, parts, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
