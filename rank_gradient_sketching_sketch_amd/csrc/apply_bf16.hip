// Apply pass 2 for bf16 compute: rebuild Ghat = S A tile by tile on the
// matrix cores and apply RowAdam, W_ij -= lr * scale * Ghat_ij / (sqrt(v'_i) + eps).
//
// The update estimate S A exists only while it is applied ("NVIDIA's LoGRA
// fits RL post-training of a 27B model onto a single eight-GPU node", section
// "Why it matters"); RowAdam keeps one running second moment per row and no
// first moment (same page, "What happened" and "Why it matters").
//
// Work decomposition. The unit of work is one row tile of W (256 rows, or
// 128 when the matrix is too small to give every workgroup at least four
// 256-row units) times one 64-column tile; the units, in row-major order,
// are dealt to a fixed number of workgroups as contiguous ranges of equal
// cost, counting the load of a row tile's S rows as a few units (one
// workgroup per compute unit), so a workgroup touches at most a few row tiles
// and loads their rows of S only once each. Neighbouring ranges (which share
// a row tile) run on the same XCD, so S is fetched from HBM about once and
// the other workgroups of the row tile find it in that XCD's L2. Eight waves
// (two per SIMD, so one wave's vector work overlaps the other's matrix work)
// each own 32 (or 16) of the tile's rows and keep S^T for them as bf16 MFMA
// operands in registers. The 128-row tiles halve the S a workgroup loads for
// its few units (1536 x 1536: 13.5 instead of 18.9 us per call).
//
// Per column tile: every thread hashes one 64-bit sign word (rank row l,
// these 64 columns) into LDS; each wave then builds an eighth of the tile's
// 32 sign fragments (16 columns x 32 rank indices, bf16 +-1) from the words
// and stores them to LDS, so every fragment is built once per workgroup and
// read by all eight waves. The MFMA computes Ghat^T tiles (A = signs, B =
// S^T); MFMA row m of pseudo column block cb stands for column
// 32 (cb / 2) + 8 (m / 4) + 4 (cb % 2) + m % 4, which puts 8 consecutive
// columns of one row of W in each lane, so W moves in 16-byte vectors. W
// goes through a buffer view (rows past d and columns past k read as zero
// and are not written) and is requested one tile ahead of its products (two
// ahead of its update, which lags the products by one unit).
//
// u_i comes from the updated second moment v' that pass 1 wrote; nothing
// but W is written, so the same kernel rebuilds the update on any replica
// of W that receives S and v'.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

constexpr uint32_t kOobOff = 0x80000000u;
constexpr int kApplyRowsMax = 256;     // rows of W per row tile, most (32 per wave)
constexpr int kApplyWaves = 8;
constexpr int kApplyCols = 64;         // columns per column tile (one sign word)
constexpr int kApplyWGs = 256;         // workgroups (one per compute unit)

// With more than one apply call in flight at once on separate streams (the
// caller's apply_concurrency launch option), pass 2 of a large matrix (at
// least kConcurrentMinUnits 256-row units) deals its units over half as
// many workgroups, which then walk longer ranges while the other streams
// fill the rest of the chip; smaller matrices measured slower that way and
// keep the full grid.
constexpr int64_t kConcurrentMinUnits = 1024;

static int apply_wgs(int64_t units256, int concurrency) {
    return concurrency > 1 && units256 >= kConcurrentMinUnits ? kApplyWGs / 2 : kApplyWGs;
}
constexpr int kTallTileUnitsPerWG = 4;  // 256-row units per workgroup from which 256-row tiles are used
constexpr int kStagePitch = 144;       // bytes per staged row of a wave's updated bf16 block

// Barrier that orders LDS traffic only (global loads stay in flight).
__device__ __forceinline__ void apply_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int R, bool WBF16, int RB>
__global__ __launch_bounds__(512) void rowadam_bf16_kernel(ApplyArgs a, int n_ct, int n_units) {
    constexpr int kApplyRows = 128 * RB;       // rows of W per row tile (16 RB per wave)
    constexpr int WR = 16 * RB;                // rows per wave
    constexpr int KS = R / 32;                 // 32-wide steps of the rank
    constexpr int WV = WBF16 ? 1 : 2;          // 16-byte vectors per 8 columns of W
    constexpr int NF = 4 * KS;                 // sign fragments per column tile
    __shared__ uint32_t words[2][2][R];        // [buffer][half of the 64 columns][l]
    __shared__ __attribute__((aligned(16))) u32x4_t frags[2][NF][64];   // [buffer][fragment][lane]
    __shared__ float coef_s[kApplyRows];
    // bf16 W: each wave's updated 32 x 64 block on its way from the MFMA
    // layout to whole-line stores (rows padded to 144 bytes: conflict-free
    // both ways)
    __shared__ __attribute__((aligned(16))) uint8_t wstage[WBF16 ? kApplyWaves * WR * kStagePitch : 16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int D = static_cast<int>(a.D), K = static_cast<int>(a.K);

    // workgroup ids are dealt round-robin over the 8 XCDs
    const int G = gridDim.x;
    const int range = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : static_cast<int>(blockIdx.x);
    // The ranges have equal cost rather than equal length: each row tile
    // costs its n_ct units plus kTileCost more for loading its rows of S (the
    // bytes of S per row tile over the bytes of W one unit reads and writes),
    // so a range that starts a new row tile is that much shorter.
    constexpr int kTileCost = (R * 4) / (kApplyCols * 2 * (WBF16 ? 2 : 4)) > 1
                                  ? (R * 4) / (kApplyCols * 2 * (WBF16 ? 2 : 4))
                                  : 1;
    const int64_t per_tile = n_ct + kTileCost;
    const int64_t total = static_cast<int64_t>(n_units / n_ct) * per_tile;
    auto unit_at = [&](int64_t cpos) -> int {   // first unit at or after cost position cpos
        const int64_t t = cpos / per_tile;
        int64_t j = cpos - t * per_tile - kTileCost;
        if (j < 0) j = 0;
        const int64_t u = t * n_ct + j;
        return static_cast<int>(u < n_units ? u : n_units);
    };
    const int u_begin = unit_at(static_cast<int64_t>(range) * total / G);
    const int u_end = unit_at(static_cast<int64_t>(range + 1) * total / G);

    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.W, 0, static_cast<int>(static_cast<int64_t>(D) * a.ldw * (WBF16 ? 2 : 4)), 0x00020000);
    // Position of a unit: row tile, column tile (advanced one unit at a time).
    struct Pos {
        int u, rt, ct;
    };
    auto advance = [&](Pos p) -> Pos {
        ++p.u;
        if (++p.ct == n_ct) {
            p.ct = 0;
            ++p.rt;
        }
        return p;
    };
    // Byte offset of lane (n, g)'s 8 columns of row block rb, column half h,
    // in unit p (kOobOff if masked).
    auto w_off = [&](const Pos &p, int rb, int h) -> uint32_t {
        const int i = p.rt * kApplyRows + WR * wave + 16 * rb + n;
        const int jc = p.ct * kApplyCols + 32 * h + 8 * g;
        const bool ok = p.u < u_end && i < D && jc < K;
        return ok ? static_cast<uint32_t>((static_cast<int64_t>(i) * a.ldw + jc) * (WBF16 ? 2 : 4)) : kOobOff;
    };
    auto w_load = [&](const Pos &p, u32x4_t (&w)[RB][2][WV]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t off = w_off(p, rb, h);
#pragma unroll
                for (int x = 0; x < WV; ++x)
                    w[rb][h][x] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                  w_rs, off == kOobOff ? off : off + 16 * x, 0, 0));
            }
    };
    // Sign words of unit p: thread l (< R) hashes rank row l, word block ct.
    auto hash_words = [&](const Pos &p, int buf) {
        if (tid < R && p.u < u_end) {
            const uint64_t w = sign_word(a.key, static_cast<uint32_t>(tid), static_cast<uint32_t>(p.ct));
            words[buf][0][tid] = static_cast<uint32_t>(w);
            words[buf][1][tid] = static_cast<uint32_t>(w >> 32);
        }
    };
    // Fragment (cb, s), lane (n, g): rank rows l = 32 s + 8 g + e (e = 0..7),
    // column 32 (cb / 2) + 8 (n / 4) + 4 (cb % 2) + n % 4; element e is
    // +-1 in bf16, element pairs packed low half first. Wave w builds the
    // fragments of steps s with s % 8 == w.
    const int jbit = 8 * (n >> 2) + (n & 3);
    auto build_step = [&](int buf, int s) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t w0 = *reinterpret_cast<const u32x4_t *>(&words[buf][h][32 * s + 8 * g]);
            const u32x4_t w1 = *reinterpret_cast<const u32x4_t *>(&words[buf][h][32 * s + 8 * g + 4]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const uint32_t sh = jbit + 4 * mb;
                u32x4_t f;
                f.x = __builtin_amdgcn_ubfe(w0.y, sh, 1) << 31 | __builtin_amdgcn_ubfe(w0.x, sh, 1) << 15 | 0x3F803F80u;
                f.y = __builtin_amdgcn_ubfe(w0.w, sh, 1) << 31 | __builtin_amdgcn_ubfe(w0.z, sh, 1) << 15 | 0x3F803F80u;
                f.z = __builtin_amdgcn_ubfe(w1.y, sh, 1) << 31 | __builtin_amdgcn_ubfe(w1.x, sh, 1) << 15 | 0x3F803F80u;
                f.w = __builtin_amdgcn_ubfe(w1.w, sh, 1) << 31 | __builtin_amdgcn_ubfe(w1.z, sh, 1) << 15 | 0x3F803F80u;
                frags[buf][(2 * h + mb) * KS + s][lane] = f;
            }
        }
    };
    auto build_frags = [&](int buf) {
        if constexpr (KS % kApplyWaves == 0) {
#pragma unroll
            for (int j = 0; j < KS / kApplyWaves; ++j) build_step(buf, wave + kApplyWaves * j);
        } else {
            for (int s = wave; s < KS; s += kApplyWaves) build_step(buf, s);
        }
    };

    // S^T fragments of the current row tile: lane (n, g) of row block rb,
    // step s holds S[i][32 s + 8 g .. +7] in bf16, i = row 32 wave + 16 rb + n
    // of the tile (rows past d are clamped: their products are never stored).
    u32x4_t sf[RB][KS];
    int cur_rt = -1;
    auto load_rows = [&](int rt) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int i = min(rt * kApplyRows + WR * wave + 16 * rb + n, D - 1);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const float *p = a.S + static_cast<int64_t>(i) * R + 32 * s + 8 * g;
                const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p);
                const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(p + 4);
                sf[rb][s] = u32x4_t{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                                    pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
            }
        }
        // u_i for the 256 rows, with the c of A folded in
        if (tid < kApplyRows) {
            const int i = rt * kApplyRows + tid;
            float coef = 0.f;
            if (i < D) {
                coef = a.lr_scale * a.c / (sqrtf(a.v_new_in[i]) + a.eps);
            }
            coef_s[tid] = coef;
        }
        cur_rt = rt;
    };

    // W_ij -= cf_i * (Ghat/c)_ij for the unit at p: lane (n, g) of (rb, cb)
    // holds row 32 wave + 16 rb + n, columns 32 (cb / 2) + 8 g + 4 (cb % 2) .. +3.
    auto finish = [&](const f32x4_t (&acc)[RB][4], const float (&cf)[RB], const Pos &p,
                      const u32x4_t (&wv)[RB][2][WV]) {
        if (WBF16) {
            // The MFMA layout gives each lane 16 bytes of one row, so a wave's
            // store would cover 16 rows x 64 bytes (half cache lines). The
            // wave writes its block to LDS instead and stores it back as 8
            // rows x 128 bytes per instruction (lane L: row 8 q + L / 8,
            // columns 8 (L % 8) .. +7), whole lines, which HBM takes much
            // faster.
            uint8_t *blk = wstage + wave * WR * kStagePitch;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4_t x0 = acc[rb][2 * h], x1 = acc[rb][2 * h + 1];
                    const float c = cf[rb];
                    const u32x4_t w = wv[rb][h][0];
                    u32x4_t o;
                    o.x = pack_bf16x2(fmaf(-c, x0.x, bf16_lo(w.x)), fmaf(-c, x0.y, bf16_hi(w.x)));
                    o.y = pack_bf16x2(fmaf(-c, x0.z, bf16_lo(w.y)), fmaf(-c, x0.w, bf16_hi(w.y)));
                    o.z = pack_bf16x2(fmaf(-c, x1.x, bf16_lo(w.z)), fmaf(-c, x1.y, bf16_hi(w.z)));
                    o.w = pack_bf16x2(fmaf(-c, x1.z, bf16_lo(w.w)), fmaf(-c, x1.w, bf16_hi(w.w)));
                    *reinterpret_cast<u32x4_t *>(blk + (16 * rb + n) * kStagePitch + 64 * h + 16 * g) = o;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
            const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
            for (int q = 0; q < 2 * RB; ++q) {
                const int row = 8 * q + lr;
                const u32x4_t o = *reinterpret_cast<const u32x4_t *>(blk + row * kStagePitch + 16 * lc);
                const int i = p.rt * kApplyRows + WR * wave + row;
                const int jc = p.ct * kApplyCols + 8 * lc;
                const uint32_t off = (p.u < u_end && i < D && jc < K)
                                         ? static_cast<uint32_t>((static_cast<int64_t>(i) * a.ldw + jc) * 2)
                                         : kOobOff;
                __builtin_amdgcn_raw_buffer_store_b128(o, w_rs, off, 0, 0);
            }
            // the reads above are done before the next unit's block is written
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4_t x0 = acc[rb][2 * h], x1 = acc[rb][2 * h + 1];
                    const uint32_t off = w_off(p, rb, h);
                    const float c = cf[rb];
                    f32x4_t w0v = __builtin_bit_cast(f32x4_t, wv[rb][h][0]);
                    f32x4_t w1v = __builtin_bit_cast(f32x4_t, wv[rb][h][WV - 1]);
                    w0v.x = fmaf(-c, x0.x, w0v.x); w0v.y = fmaf(-c, x0.y, w0v.y);
                    w0v.z = fmaf(-c, x0.z, w0v.z); w0v.w = fmaf(-c, x0.w, w0v.w);
                    w1v.x = fmaf(-c, x1.x, w1v.x); w1v.y = fmaf(-c, x1.y, w1v.y);
                    w1v.z = fmaf(-c, x1.z, w1v.z); w1v.w = fmaf(-c, x1.w, w1v.w);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w0v), w_rs, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w1v), w_rs,
                                                          off == kOobOff ? off : off + 16, 0, 0);
                }
        }
    };

    if (u_begin >= u_end) return;
    Pos p0;   // the unit whose products are formed
    p0.u = u_begin;
    p0.rt = u_begin / n_ct;
    p0.ct = u_begin - p0.rt * n_ct;
    Pos pp = p0;    // the unit whose update is written (one behind p0)
    pp.u = u_end;   // none yet: w_off masks every access of a unit >= u_end
    Pos p1 = advance(p0);   // the unit whose W is requested
    Pos p2 = advance(p1);   // the unit whose sign words are requested
    u32x4_t wb[2][RB][2][WV];   // W ring: slot (u - u_begin) % 2 holds unit u
    w_load(p0, wb[0]);
    hash_words(p0, 0);
    apply_lds_barrier();
    build_frags(0);
    hash_words(p1, 1);
    f32x4_t prev[RB][4];
    float cf_prev[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) cf_prev[rb] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) prev[rb][cb] = zero_f32x4();

    // Software pipeline, one unit per step: the products of unit u, the
    // update of unit u - 1 and the sign fragments of unit u + 1 share one
    // straight-line block, so the matrix cores and the vector units work at
    // the same time. Units go in pairs so the W ring index (two slots) is a
    // compile-time constant.
    for (int u0 = u_begin; u0 < u_end; u0 += 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int u = u0 + p;
            if (u < u_end) {
                const int buf = (u - u_begin) & 1;
                if (p0.rt != cur_rt) {
                    // every wave is done with the previous row tile's coef_s
                    __syncthreads();
                    load_rows(p0.rt);
                }
                apply_lds_barrier();   // fragments of u and words of u + 1 are in LDS
                f32x4_t acc[RB][4];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = zero_f32x4();
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        const u32x4_t af = frags[buf][cb * KS + s][lane];
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) acc[rb][cb] = mfma_bf16(af, sf[rb][s], acc[rb][cb]);
                    }
                float cf_cur[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) cf_cur[rb] = coef_s[WR * wave + 16 * rb + n];
                finish(prev, cf_prev, pp, wb[(p + 1) % 2]);   // unit u - 1 (slot (u - 1) % 2)
                w_load(p1, wb[(p + 1) % 2]);                 // unit u + 1 into the freed slot
                build_frags(buf ^ 1);
                hash_words(p2, buf);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    cf_prev[rb] = cf_cur[rb];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) prev[rb][cb] = acc[rb][cb];
                }
                pp = p0;
                p0 = advance(p0);
                p1 = advance(p1);
                p2 = advance(p2);
            }
        }
    }
    // the last unit's update: slot (u_end - 1 - u_begin) % 2
    if ((u_end - 1 - u_begin) % 2 == 0)
        finish(prev, cf_prev, pp, wb[0]);
    else
        finish(prev, cf_prev, pp, wb[1]);
}

template <int R, int RB>
static hipError_t rowadam_rb(const ApplyArgs &a, int wgs, hipStream_t st) {
    constexpr int rows = 128 * RB;
    const int n_rt = static_cast<int>((a.D + rows - 1) / rows);
    const int n_ct = static_cast<int>((a.K + kApplyCols - 1) / kApplyCols);
    const int n_units = n_rt * n_ct;
    const int grid = n_units < wgs ? n_units : wgs;
    if (a.w_bf16)
        hipLaunchKernelGGL((rowadam_bf16_kernel<R, true, RB>), dim3(grid), dim3(64 * kApplyWaves), 0, st, a, n_ct,
                           n_units);
    else
        hipLaunchKernelGGL((rowadam_bf16_kernel<R, false, RB>), dim3(grid), dim3(64 * kApplyWaves), 0, st, a, n_ct,
                           n_units);
    return hipGetLastError();
}

// Row tiles of 256 rows when each workgroup gets enough units of them to
// amortise loading its rows of S (256 KB at r = 256), otherwise 128 rows,
// which halve that load at the price of sign fragments shared by fewer rows.
template <int R>
static hipError_t rowadam_r(const ApplyArgs &a, int concurrency, hipStream_t st) {
    const int64_t units256 = ((a.D + kApplyRowsMax - 1) / kApplyRowsMax) * ((a.K + kApplyCols - 1) / kApplyCols);
    const int wgs = apply_wgs(units256, concurrency);
    if (units256 >= static_cast<int64_t>(kTallTileUnitsPerWG) * wgs) return rowadam_rb<R, 2>(a, wgs, st);
    return rowadam_rb<R, 1>(a, wgs, st);
}

hipError_t launch_rowadam_bf16(const ApplyArgs &a, int concurrency, hipStream_t st) {
    switch (a.R) {
    case 32: return rowadam_r<32>(a, concurrency, st);
    case 64: return rowadam_r<64>(a, concurrency, st);
    case 128: return rowadam_r<128>(a, concurrency, st);
    case 256: return rowadam_r<256>(a, concurrency, st);
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
