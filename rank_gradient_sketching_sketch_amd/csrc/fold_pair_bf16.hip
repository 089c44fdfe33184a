// The pair-mode instances of the fold kernel (fold_bf16.hip describes the
// fold; fold_body.hpp holds its body): two members per tile that add their
// partials inside the launch. They are built here, with the accumulators in
// the accumulation registers, because the vector-register form that the
// other instances are built with made them about 3 % slower.
#include "fold_body.hpp"

namespace logra {

template <int R>
static hipError_t pair_r(int max_blocks, int n_wg, hipStream_t st, const uint16_t *dY, int64_t lddy, int T, int D,
                         const uint16_t *P, int p_blocks, float *S, float *xbuf, int x_bytes, int *sync,
                         int accumulate, int nblk, int n_tiles, int n_split, int steps_per, int spin_limit,
                         int *timeouts) {
    auto kernel = max_blocks == 5 ? fold_bf16_kernel<R, 5, kFoldPair> : fold_bf16_kernel<R, 10, kFoldPair>;
    hipLaunchKernelGGL(kernel, dim3(n_wg), dim3(256), 0, st, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync,
                       accumulate, nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
    return hipGetLastError();
}

hipError_t launch_fold_pair_bf16(int R, int max_blocks, int n_wg, hipStream_t st, const uint16_t *dY,
                                 int64_t lddy, int T, int D, const uint16_t *P, int p_blocks, float *S,
                                 float *xbuf, int x_bytes, int *sync, int accumulate, int nblk, int n_tiles,
                                 int n_split, int steps_per, int spin_limit, int *timeouts) {
    switch (R) {
    case 32:
        return pair_r<32>(max_blocks, n_wg, st, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync, accumulate,
                          nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
    case 64:
        return pair_r<64>(max_blocks, n_wg, st, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync, accumulate,
                          nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
    case 128:
        return pair_r<128>(max_blocks, n_wg, st, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync, accumulate,
                           nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
    case 256:
        return pair_r<256>(max_blocks, n_wg, st, dY, lddy, T, D, P, p_blocks, S, xbuf, x_bytes, sync, accumulate,
                           nblk, n_tiles, n_split, steps_per, spin_limit, timeouts);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace logra
