// Peak probes for bench.py (measurement only, not part of libqlora): a
// bf16 MFMA throughput loop and a streaming copy, so that the roofline
// fractions can be read against what this GPU sustains as well as against
// the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Every wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16
// (8 accumulator chains hide the matrix core's result latency).  The sum of
// the accumulators is stored only if it equals a value it never takes, so
// the loop is kept but nothing is written.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  const int l = threadIdx.x;
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((l + i) & 7);
    b[i] = (__bf16)(float)((l * 3 + i) & 7);
  }
  f32x16_t acc[8];
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == -1.0f) out[blockIdx.x * 256 + l] = s;
}

// 16 bytes per lane per iteration, grid-stride.
__global__ __launch_bounds__(256) void copy_peak_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

extern "C" {

// Flops of one mfma_peak launch: blocks * 4 waves * iters * 8 * 32*32*16*2.
int qlora_peak_mfma(int blocks, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

// Copies bytes (a multiple of 16) from src to dst.
int qlora_peak_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(copy_peak_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
