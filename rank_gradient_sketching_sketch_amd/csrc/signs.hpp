// Counter-hash regeneration of the random-sign projection.
//
// LoGRA's projection is a random-sign r x k matrix, redrawn each optimizer
// step and held fixed across that step's microbatches ("LoGRA: Scaling LLM
// Reinforcement Learning with Low-Rank Gradient Sketches", paragraph
// "Gradient sketches."). It is never stored: every kernel recomputes the
// 64-bit words it needs. Word (l, b) carries the signs of row l, columns
// 64b .. 64b+63 (bit j mod 64; a set bit means -1). It is output number
// ((l << 32) | b) + 1 of a SplitMix64 stream (Steele, Lea & Flood, OOPSLA
// 2014) started at the per-(seed, step, matrix) key; the host derives the
// key (see stream_key in api.hip).
#pragma once

#include <stdint.h>

namespace logra {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t splitmix_finalize(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

__host__ __device__ __forceinline__ uint64_t sign_word(uint64_t key, uint32_t l, uint32_t b) {
    const uint64_t counter = ((static_cast<uint64_t>(l) << 32) | b) + 1ull;
    return splitmix_finalize(key + counter * kGolden);
}

}  // namespace logra
