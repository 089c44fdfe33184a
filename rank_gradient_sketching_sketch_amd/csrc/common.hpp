// Shared device helpers for the LoGRA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D = A(16x32 bf16) * B(32x16 bf16) + C on the matrix cores. Lane L holds
// A[L%16][8*(L/16) .. +7], B[8*(L/16) .. +7][L%16] (eight bf16 in four
// dwords, low half first) and D[4*(L/16) .. +3][L%16].
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even: one v_cvt_pk_bf16_f32
// (built as a two-element vector so both halves convert in one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Low 16-bit halves of two dwords -> one dword (lo from `lo`, hi from `hi`).
__device__ __forceinline__ uint32_t join_lo16(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
// High 16-bit halves of two dwords -> one dword.
__device__ __forceinline__ uint32_t join_hi16(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Eight sign bits x (bit e = sign of element e, 1 means -1) -> eight bf16
// +-1.0 values (0x3F80 / 0xBF80) in four dwords, element 2q in the low half
// of dword q. Only the low 8 bits of x may be set. `one` must hold 0x3F803F80
// in a register (see opaque_u32): then each dword is a shift and one
// v_and_or_b32, since a gfx9 VOP3 instruction takes no literal operand and
// with both constants as literals the compiler emits shift, and, or.
__device__ __forceinline__ u32x4_t signs8_to_bf16(uint32_t x, uint32_t one) {
    const uint32_t y = x | (x << 15);   // bit i at i and at i + 15
    u32x4_t r;
    r.x = ((y << 15) & 0x80008000u) | one;
    r.y = ((y << 13) & 0x80008000u) | one;
    r.z = ((y << 11) & 0x80008000u) | one;
    r.w = ((y << 9) & 0x80008000u) | one;
    return r;
}

// A constant in a vector register that the compiler cannot fold back into
// the instructions that use it (an empty asm statement owns it once).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ u32x4_t zero_u32x4() { return u32x4_t{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ f32x4_t zero_f32x4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ u32x4_t load_u32x4(const void *p) {
    return *reinterpret_cast<const u32x4_t *>(p);
}
__device__ __forceinline__ u32x2_t load_u32x2(const void *p) {
    return *reinterpret_cast<const u32x2_t *>(p);
}

}  // namespace logra
