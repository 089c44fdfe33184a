// Internal launchers of liblogra.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace logra {

// Work split of the first sketch product P = X A^T (bf16 path): one
// workgroup per 32 tokens and 128-column (or r-column) tile of the signs.
// P (bf16, t_blocks x r x 32) is the first thing in the sketch workspace.
struct Stage1Plan {
    int t_blocks = 0;         // 32-token blocks
    int col_tiles = 0;
    size_t p_bytes = 0;       // t_blocks * 32 * r * 2
};

Stage1Plan plan_stage1_bf16(int64_t T, int64_t K, int R);

// Work split of the fold S (+)= dY^T P (bf16 path): n_tiles row tiles over
// the nblk 16-row blocks of S, times n_split members per tile, each over
// steps_per 32-token steps. With n_split > 1 the members exchange partial
// tiles (xbuf: n_split x d x r fp32) and synchronise through sync_words ints
// (sync); both follow P in the sketch workspace.
struct FoldPlan {
    int nblk = 0;
    int n_tiles = 0;
    int n_split = 0;
    int steps_per = 0;
    int max_blocks = 0;       // 16-row blocks per tile the kernel instance is built for (5 or 10)
    int sync_words = 0;
    size_t xbuf_bytes = 0;
    size_t sync_bytes = 0;
};
// parts: the plan of the split-mode fold (logra_sketch_fold_parts), whose
// members never exchange; otherwise the plan of the fold whose members add
// their partials inside the kernel.
FoldPlan plan_fold_bf16(int64_t T, int64_t D, int R, bool parts = false);

// How a fold member waits for its partner: at most spin_limit polls
// (negative: give up at once), then its rows are written as NaN and
// *timeouts (device, may be null) is incremented.
struct FoldWait {
    int spin_limit = 1 << 20;
    int *timeouts = nullptr;
};
hipError_t launch_fold_bf16_tiles(int R, int64_t T, int64_t D, const uint16_t *dY, int64_t lddy,
                                  const uint16_t *P, int p_blocks, float *S, int accumulate,
                                  void *scratch, const FoldWait &wait, hipStream_t st);
// The pair-mode fold kernel (two members per tile adding their partials
// inside the launch) for r = R and tiles of at most max_blocks (5 or 10)
// blocks, on n_wg workgroups; the arguments are the kernel's.
hipError_t launch_fold_pair_bf16(int R, int max_blocks, int n_wg, hipStream_t st, const uint16_t *dY,
                                 int64_t lddy, int T, int D, const uint16_t *P, int p_blocks, float *S,
                                 float *xbuf, int x_bytes, int *sync, int accumulate, int nblk, int n_tiles,
                                 int n_split, int steps_per, int spin_limit, int *timeouts);
// Split-mode fold (the sketch of a step held as S plus n_split - 1 parts of
// d x r fp32): phase bit 0 starts the step (S and the parts overwritten),
// bit 1 ends it (the parts added into S afterwards, in part order).
size_t fold_parts_bytes_bf16(int64_t T, int64_t D, int R);
hipError_t launch_fold_parts_bf16(int R, int64_t T, int64_t D, const uint16_t *dY, int64_t lddy,
                                  const uint16_t *P, int p_blocks, float *S, float *parts, int phase,
                                  hipStream_t st);
// The backward input gradient dX = dY W (bf16, 256 x 256 product tiles)
// and, when sketch != 0, the fold S (+)= dY^T P in the same launch (P read
// from the projection the sketch workspace holds).
struct DxPlan {
    int n_tm = 0, n_tn = 0;       // product tiles
    int n_fold = 0;               // fold workgroups
    int fold_nblk = 0, fold_tiles = 0;
};
DxPlan plan_dx_bf16(int64_t T, int64_t D, int64_t K, int sketch);
// Whether running the fold beside the product in one launch is expected to
// be faster than the product and then the sketch's fold kernel.
bool dx_fuse_pays(int64_t T, int64_t D, int64_t K, int R);
hipError_t launch_dx_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                          const uint16_t *W, int64_t ldw, uint16_t *dX, int64_t lddx, const uint16_t *P,
                          int p_blocks, float *S, int accumulate, int sketch, const FoldWait &wait,
                          hipStream_t st);
size_t workspace_sketch_f32(int64_t T, int64_t R);
int apply_blocks_f32(int64_t D);

// Workspace of apply pass 1 with bf16 compute: one 64-bit slot per
// workgroup for its partial of the controller's reduction (a mark in the
// high word, the float's bits in the low word), then the r x r Gram matrix
// of the signs (bf16) (slots zeroed by the Gram kernel and left zero).
struct SqnormPlan {
    int n_blocks = 0;         // workgroups of rowsq_gram_kernel
    int rows_per_block = 0;   // rows of S each of them owns
    size_t partial_bytes = 0;
    size_t gram_bytes = 0;
};
SqnormPlan plan_sqnorm_bf16(int64_t D, int64_t K, int R);

hipError_t launch_sign_words(uint64_t key, int R, int K, uint64_t *words, hipStream_t st);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t st);

// stage 1: P = c X Sigma^T into the workspace (concurrency: independent
// sketch calls the caller runs at once, this one included); stage 2:
// S (+)= dY^T P from it.
hipError_t launch_project_bf16(int R, int64_t T, int64_t D, int64_t K, uint64_t key, float c,
                               const uint16_t *X, int64_t ldx, void *ws, int concurrency, hipStream_t st);
hipError_t launch_fold_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY, int64_t lddy,
                            float *S, int accumulate, void *ws, const FoldWait &wait, hipStream_t st);
// The split-mode fold reading P from the sketch workspace.
hipError_t launch_fold_parts_ws_bf16(int R, int64_t T, int64_t D, int64_t K, const uint16_t *dY,
                                     int64_t lddy, float *S, float *parts, int phase, void *ws, hipStream_t st);
hipError_t launch_project_f32(int R, int64_t T, int64_t K, uint64_t key, float c, const float *X,
                              int64_t ldx, void *ws, hipStream_t st);
hipError_t launch_fold_f32(int R, int64_t T, int64_t D, const float *dY, int64_t lddy, float *S,
                           int accumulate, const void *ws, hipStream_t st);

// Arguments of the apply passes (pointers are device pointers).
struct ApplyArgs {
    int R = 0;
    int64_t D = 0, K = 0;
    uint64_t key = 0;
    float c = 0.f;
    const float *S = nullptr;
    const float *v_in = nullptr;       // pass 1: current second moment
    float *v_new_out = nullptr;        // pass 1: updated second moment
    float *rowsq_out = nullptr;        // pass 1: row sums of squares (may be null)
    const float *v_new_in = nullptr;   // pass 2: updated second moment
    float *partials = nullptr;
    float *sqnorm = nullptr;
    float beta2 = 0.f, eps = 0.f, lr_scale = 0.f;
    void *W = nullptr;
    int w_bf16 = 0;
    int64_t ldw = 0;
};

// Pass 1 of up to kSqnormBatchMax matrices of one rank (bf16 compute), each
// with its own slice of the workspace laid out as SqnormPlan says.
constexpr int kSqnormBatchMax = 16;
struct SqnormItem {
    const float *S = nullptr;
    const float *v = nullptr;
    float *v_new = nullptr;
    float *rowsq = nullptr;        // may be null
    uint16_t *M = nullptr;         // Gram matrix in the item's workspace slice
    uint64_t *slots = nullptr;     // per-workgroup partial slots
    uint64_t key = 0;
    float c = 0.f;
    int D = 0, K = 0;
    int bpw = 0;                   // 16-row blocks per workgroup
    int wg_begin = 0, n_wg = 0;    // the item's workgroups in the batch grid
};
struct SqnormBatch {
    int n = 0;
    float beta2 = 0.f, eps = 0.f;
    float *sqnorm = nullptr;       // n floats
    SqnormItem item[kSqnormBatchMax];
};
hipError_t launch_sqnorm_batch_bf16(int R, const SqnormBatch &b, hipStream_t st);

// bf16 compute: pass 1 (Gram form, writes v', rowsq and sqnorm) and pass 2
// (RowAdam update of W from S and v').
// Pass 1 in its two kernels: the Gram matrix of the step's signs (depends
// only on the key, k and r) and the row pass that reads it.
constexpr int kSqnormGram = 1, kSqnormRows = 2;
hipError_t launch_sqnorm_bf16(const ApplyArgs &a, void *ws, hipStream_t st, int parts = kSqnormGram | kSqnormRows);
// concurrency: apply calls the caller runs at once, this one included.
hipError_t launch_rowadam_bf16(const ApplyArgs &a, int concurrency, hipStream_t st);
// fp32 compute: mode 0 = pass 1 (rowsq + partials), mode 1 = pass 2 (W and v).
hipError_t launch_apply_f32(int mode, const ApplyArgs &a, hipStream_t st);
hipError_t launch_sqnorm_final(const float *partials, int n, float *out, hipStream_t st);

// The two-sided sketch variant (rank 32, bf16 activations).
// Projection buffer of one side (n = d for P, n = k for Q): the n x 32 fp32
// orthonormal matrix, its bf16 operand copy (32-row block s, column l, row e
// at element (32 s + l) 32 + e), then scratch of its construction.
struct TsProjLayout {
    int n_blocks = 0;
    size_t fp32_bytes = 0, frag_bytes = 0, z_bytes = 0, partial_bytes = 0, gram_bytes = 0, rinv_bytes = 0;
    size_t total = 0;
};
TsProjLayout ts_projection_layout(int64_t n);
hipError_t launch_ts_projection(uint64_t key, int64_t n, void *buf, hipStream_t st);
// Sketch workspace: Xq and Yp (bf16, fold operand layout), the fp32 partials
// of the projection kernel, then the scratch of each of the two folds.
struct TsSketchLayout {
    int p_blocks = 0;
    int chunks[2] = {0, 0};           // column chunks of X (job 0) and dY (job 1)
    size_t p_bytes = 0, part_bytes = 0;
    FoldPlan fold[2];                 // S_R over d, S_L^T over k
    size_t fold_off[2] = {0, 0};
    size_t total = 0;
};
TsSketchLayout ts_sketch_layout(int64_t T, int64_t d, int64_t k);
hipError_t launch_ts_sketch(int64_t T, int64_t d, int64_t k, const uint16_t *X, int64_t ldx, const uint16_t *dY,
                            int64_t lddy, const void *projP, const void *projQ, float *S_L, float *S_R,
                            int accumulate, void *ws, const FoldWait &wait, hipStream_t st);
// Update workspace: U_R, U_L, B = U_R C, C, the three summed Gram matrices,
// the per-block partials. It holds what the apply call reads.
struct TsUpdateLayout {
    int nr = 0, nl = 0;
    size_t ur_off = 0, ul_off = 0, b_off = 0, c_off = 0, sums_off = 0, partial_off = 0, total = 0;
};
TsUpdateLayout ts_update_layout(int64_t d, int64_t k);
hipError_t launch_ts_update(int64_t d, int64_t k, const float *S_L, const float *S_R, const void *projP, float *m_L,
                            float *v_L, float *m_R, float *v_R, float beta1, float beta2, float eps, float *sqnorm,
                            void *ws, hipStream_t st);
hipError_t launch_ts_apply(int64_t d, int64_t k, const void *ws, void *W, int w_bf16, int64_t ldw, float step,
                           hipStream_t st);

}  // namespace logra
