// Shared device helpers for the gfx950 kernels of libqlora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace qlora {

constexpr int kBlock = 64;    // weights per absmax block
constexpr int kBlock2 = 256;  // absmax constants per second-level group

// The NF4 table and its decision boundaries travel to kernels by value.
struct Codebook {
  float c[16];
};
struct Midpoints {
  double m[15];
};

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
// `lo` lands in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Dequantized first-level constant fp32(q8 * s2 / 255), rounded once.
// q8*s2 is exact in fp64; multiplying by the fp64 reciprocal of 255 adds at
// most 2^-52 relative error, while q8*s2/255 is never closer than 2^-33
// (relative) to an fp32 halfway point, so the final fp32 rounding is the
// correct one.
__device__ __forceinline__ float dq_scale(uint32_t q8, float s2) {
  return (float)((double)q8 * (double)s2 * (1.0 / 255.0));
}

}  // namespace qlora
