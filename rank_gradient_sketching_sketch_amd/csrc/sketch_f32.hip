// Sketch accumulation S (+)= dY^T (X A^T) in fp32 (no reduced-precision
// products), for fp32 activations. Same two products as the bf16 path
// ("NVIDIA's LoGRA fits RL post-training...", section "Why it matters"):
// stage 1 P = c * X Sigma^T with the signs regenerated from the counter hash,
// stage 2 S (+)= dY^T P. Plain LDS-tiled fp32 FMA kernels; every sum runs in
// index order inside one thread, so results are deterministic.
#include "common.hpp"
#include "launch.hpp"
#include "signs.hpp"

namespace logra {

// P[t][l] = c * sum_j X[t][j] * sigma(l, j). Tile: 32 tokens x 32 columns of r.
__global__ __launch_bounds__(256) void stage1_f32_kernel(const float *__restrict__ X, int64_t ldx,
                                                         int T, int K, int R, uint64_t key, float c,
                                                         float *__restrict__ P) {
    __shared__ float xs[32][65];
    __shared__ uint64_t wsg[32];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int t0 = blockIdx.x * 32, l0 = blockIdx.y * 32;
    const int l = l0 + tx;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < K; j0 += 64) {
        for (int e = 0; e < 8; ++e) {
            const int idx = threadIdx.x + 256 * e;
            const int tt = idx >> 6, jj = idx & 63;
            const int t = t0 + tt, j = j0 + jj;
            xs[tt][jj] = (t < T && j < K) ? X[static_cast<int64_t>(t) * ldx + j] : 0.f;
        }
        if (threadIdx.x < 32) {
            const int ll = l0 + threadIdx.x;
            wsg[threadIdx.x] = ll < R ? sign_word(key, static_cast<uint32_t>(ll),
                                                  static_cast<uint32_t>(j0 >> 6))
                                      : 0ull;
        }
        __syncthreads();
        const uint64_t w = wsg[tx];
        const int jn = min(64, K - j0);
        for (int jj = 0; jj < jn; ++jj) {
            const float sg = ((w >> jj) & 1ull) ? -1.f : 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(sg, xs[ty + 8 * q][jj], acc[q]);
        }
        __syncthreads();
    }
    if (l < R) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = t0 + ty + 8 * q;
            if (t < T) P[static_cast<int64_t>(t) * R + l] = c * acc[q];
        }
    }
}

// S[i][l] (+)= sum_t dY[t][i] * P[t][l]. Tile: 32 rows x 32 columns of r.
__global__ __launch_bounds__(256) void stage2_f32_kernel(const float *__restrict__ dY, int64_t lddy,
                                                         int T, int D, int R,
                                                         const float *__restrict__ P,
                                                         float *__restrict__ S, int accumulate) {
    __shared__ float ds[32][33];
    __shared__ float ps[32][33];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int i0 = blockIdx.x * 32, l0 = blockIdx.y * 32;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < T; t0 += 32) {
        for (int e = 0; e < 4; ++e) {
            const int idx = threadIdx.x + 256 * e;
            const int tt = idx >> 5, cc = idx & 31;
            const int t = t0 + tt;
            ds[tt][cc] = (t < T && i0 + cc < D) ? dY[static_cast<int64_t>(t) * lddy + i0 + cc] : 0.f;
            ps[tt][cc] = (t < T && l0 + cc < R) ? P[static_cast<int64_t>(t) * R + l0 + cc] : 0.f;
        }
        __syncthreads();
        const int tn = min(32, T - t0);
        for (int tt = 0; tt < tn; ++tt) {
            const float p = ps[tt][tx];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(ds[tt][ty + 8 * q], p, acc[q]);
        }
        __syncthreads();
    }
    const int l = l0 + tx;
    if (l < R) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + ty + 8 * q;
            if (i < D) {
                float *dst = S + static_cast<int64_t>(i) * R + l;
                *dst = (accumulate ? *dst : 0.f) + acc[q];
            }
        }
    }
}

size_t workspace_sketch_f32(int64_t T, int64_t R) { return static_cast<size_t>(T) * R * 4; }

hipError_t launch_project_f32(int R, int64_t T, int64_t K, uint64_t key, float c, const float *X,
                              int64_t ldx, void *ws, hipStream_t st) {
    float *P = static_cast<float *>(ws);
    hipLaunchKernelGGL(stage1_f32_kernel, dim3((T + 31) / 32, (R + 31) / 32), dim3(256), 0, st, X,
                       ldx, static_cast<int>(T), static_cast<int>(K), R, key, c, P);
    return hipGetLastError();
}

hipError_t launch_fold_f32(int R, int64_t T, int64_t D, const float *dY, int64_t lddy, float *S,
                           int accumulate, const void *ws, hipStream_t st) {
    const float *P = static_cast<const float *>(ws);
    hipLaunchKernelGGL(stage2_f32_kernel, dim3((D + 31) / 32, (R + 31) / 32), dim3(256), 0, st, dY,
                       lddy, static_cast<int>(T), static_cast<int>(D), R, P, S, accumulate);
    return hipGetLastError();
}

// ------------------------------------------------------------ small kernels --
__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

__global__ void sign_words_kernel(uint64_t key, int R, int NB, uint64_t *words) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < static_cast<int64_t>(R) * NB)
        words[i] = sign_word(key, static_cast<uint32_t>(i / NB), static_cast<uint32_t>(i % NB));
}

hipError_t launch_sign_words(uint64_t key, int R, int K, uint64_t *words, hipStream_t st) {
    const int nb = (K + 63) / 64;
    const int64_t n = static_cast<int64_t>(R) * nb;
    hipLaunchKernelGGL(sign_words_kernel, dim3((n + 255) / 256), dim3(256), 0, st, key, R, nb, words);
    return hipGetLastError();
}

}  // namespace logra
