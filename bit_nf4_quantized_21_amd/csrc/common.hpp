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
// Decision data of a stored 4-bit type: the boundaries between its sorted
// distinct levels (exact in fp64; +inf past the type's last), the code of
// sorted level i in bits 4i..4i+3 of `codes`, and the code of the value 0.
struct Midpoints {
  double m[15];
  uint64_t codes;
  uint32_t zero_code;
};
__host__ __device__ __forceinline__ uint32_t level_code(const Midpoints& mp, uint32_t level) {
  return (uint32_t)(mp.codes >> (4 * level)) & 15u;
}

// Writes the codebook to lut[0..15] (16-byte aligned) from thread 0 with
// four vector stores of the kernel argument's values.  No lane-indexed read
// of the argument is issued: such a read is a memory load that would wait for
// every load issued before it.
__device__ __forceinline__ void codebook_to_lds(float* lut, const Codebook& cb, int tid) {
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<float4*>(lut)[q] = make_float4(cb.c[4 * q], cb.c[4 * q + 1], cb.c[4 * q + 2], cb.c[4 * q + 3]);
  }
}

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

// Decode 8 NF4 codes (one dword; element 2i in the low nibble of byte i) with
// the per-block scale into 8 bf16 weights, packed as 4 bf16 pairs: the
// compute weight bf16(c[code] * scale) of the dequantization rule.  `lut` is
// the 16-entry fp32 codebook in LDS (16 distinct banks: conflict-free).
__device__ __forceinline__ void decode8_bf16(uint32_t x, float sc, const float* lut, uint32_t out[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t b = x >> (8 * p);
    out[p] = pack_bf16x2(lut[b & 15u] * sc, lut[(b >> 4) & 15u] * sc);
  }
}

// Same decode to fp32 values (one fp32 multiply each, before bf16 rounding).
__device__ __forceinline__ void decode8_f32(uint32_t x, float sc, const float* lut, float out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = lut[(x >> (4 * e)) & 15u] * sc;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Split fp32 values into bf16 hi + lo parts (v ~= hi + lo to ~16 bits) so that
// two bf16 MFMAs reproduce an fp32 operand to about 2^-17 relative.
__device__ __forceinline__ void split_bf16x8(const float v[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
    l[p] = pack_bf16x2(v[2 * p] - bf16_lo(h[p]), v[2 * p + 1] - bf16_hi(h[p]));
  }
  hi = as_bf16x8(h[0], h[1], h[2], h[3]);
  lo = as_bf16x8(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float v[8]) {
  return as_bf16x8(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer descriptors: loads at offsets at or past `bytes` return zero, so
// ragged tile edges need no branches.  Offsets are 32-bit, relative to base;
// kOffNone is past every view (a masked lane loads zero without a branch).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffNone = 0x7FFFFF00u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// `off` where ok, else kOffNone, without a branch: the lane mask passes
// through an empty asm, so the optimizer cannot turn the choice back into
// control flow around the load that uses it.
__device__ __forceinline__ uint32_t off_if(bool ok, uint32_t off) {
  uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return (off & m) | (kOffNone & ~m);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Asynchronous copy of 16 bytes per lane from a buffer straight into LDS
// (buffer_load_dwordx4 ... lds): lane i of the wave writes the 16 bytes at
// byte offset `off` of the buffer to lds_block + 16 * i.  Completion is
// tracked by vmcnt like any buffer load.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void buf_load16_to_lds(rsrc_t r, void* lds_block, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_block, 16, (int)off, 0, 0, 0);
}

// v_bfe_u32 with constant offset / width, kept as one instruction (the
// compiler otherwise splits some extracts into a shift and a mask).
template <int OFF, int W>
__device__ __forceinline__ uint32_t bfe(uint32_t x) {
  uint32_t r;
  asm("v_bfe_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "i"(OFF), "i"(W));
  return r;
}

// Byte q (0..3, a constant once unrolled) of x, by one v_bfe_u32.
__device__ __forceinline__ uint32_t bfe8(uint32_t x, int q) {
  switch (q) {
    case 0: return bfe<0, 8>(x);
    case 1: return bfe<8, 8>(x);
    case 2: return bfe<16, 8>(x);
    default: return bfe<24, 8>(x);
  }
}

// Codebook values of the 8 codes of a dword, element e = nibble e, from the
// 16-entry fp32 table at LDS address 0 (`lds` points there): byte q of
// (x << 2) & 0x3C3C3C3C is 4 * code(2q), of (x >> 2) & 0x3C3C3C3C is
// 4 * code(2q + 1), so each lookup address is one bitfield extract.
__device__ __forceinline__ void lut8_lds0(const unsigned char* lds, uint32_t x, float (&f)[8]) {
  const uint32_t y4 = (x << 2) & 0x3C3C3C3Cu, z4 = (x >> 2) & 0x3C3C3C3Cu;
  f[0] = *reinterpret_cast<const float*>(lds + bfe<0, 8>(y4));
  f[1] = *reinterpret_cast<const float*>(lds + bfe<0, 8>(z4));
  f[2] = *reinterpret_cast<const float*>(lds + bfe<8, 8>(y4));
  f[3] = *reinterpret_cast<const float*>(lds + bfe<8, 8>(z4));
  f[4] = *reinterpret_cast<const float*>(lds + bfe<16, 8>(y4));
  f[5] = *reinterpret_cast<const float*>(lds + bfe<16, 8>(z4));
  f[6] = *reinterpret_cast<const float*>(lds + bfe<24, 8>(y4));
  f[7] = *reinterpret_cast<const float*>(lds + bfe<24, 8>(z4));
}

// 8 * byte q of x (q = 0..3, a constant once unrolled) in one VALU
// instruction: a shift whose source operand selects the byte (SDWA).
template <int Q>
__device__ __forceinline__ uint32_t byte_x8(uint32_t x) {
  uint32_t r;
  if constexpr (Q == 0)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(x));
  else if constexpr (Q == 1)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(x));
  else if constexpr (Q == 2)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(x));
  else
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ uint32_t byte_x8(uint32_t x, int q) {
  switch (q) {
    case 0: return byte_x8<0>(x);
    case 1: return byte_x8<1>(x);
    case 2: return byte_x8<2>(x);
    default: return byte_x8<3>(x);
  }
}

// Pair table of the codebook at LDS address 0: entry b (b = one code byte,
// element 2q in its low nibble) holds (c[b & 15], c[b >> 4]), so one 8-byte
// LDS read returns the codebook values of two consecutive elements and its
// address is 8 * b.  Built from the 16-entry codebook at `lut16` (already in
// LDS and visible) by the workgroup's first 256 threads; the caller makes
// the table visible with a barrier.
__device__ __forceinline__ void pair_table_to_lds(unsigned char* lds, const float* lut16, int tid) {
  if (tid < 256) reinterpret_cast<float2*>(lds)[tid] = make_float2(lut16[tid & 15], lut16[tid >> 4]);
}
// The same table built from the kernel argument by lane selects.  The
// values pass through an empty asm first, so the selects cannot be folded
// into a lane-indexed read of the argument (a memory load that would wait
// for every load issued before it).
__device__ __forceinline__ void pair_table_from_arg(unsigned char* lds, const Codebook& cb, int tid) {
  if (tid < 256) {
    float c[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      c[e] = cb.c[e];
      asm volatile("" : "+v"(c[e]));
    }
    const uint32_t lo = tid & 15, hi = tid >> 4;
    float a = c[0], b = c[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      a = lo == (uint32_t)e ? c[e] : a;
      b = hi == (uint32_t)e ? c[e] : b;
    }
    reinterpret_cast<float2*>(lds)[tid] = make_float2(a, b);
  }
}
// Codebook values of the 8 codes of a dword from the pair table.
__device__ __forceinline__ void lut8_pairs(const unsigned char* lds, uint32_t x, float (&f)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float2 v = *reinterpret_cast<const float2*>(lds + byte_x8(x, q));
    f[2 * q] = v.x;
    f[2 * q + 1] = v.y;
  }
}

// Workgroup barrier that waits for this wave's LDS operations only (global
// loads stay in flight across it).  The memory clobber keeps the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace qlora
