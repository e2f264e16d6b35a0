// Launchers of the gfx950 kernels (host side, enqueue on `s`, no sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

struct Codebook;
struct Midpoints;

hipError_t launch_quantize_nf4(const float* W, int64_t n, uint8_t* codes, float* absmax,
                               const Midpoints& mp, hipStream_t s);
hipError_t launch_quantize_nf4_bf16(const uint16_t* W, int64_t n, uint8_t* codes, float* absmax,
                                    const Midpoints& mp, hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* q8, float* s2, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                             int out_bf16, void* out, const Codebook& cb, hipStream_t s);

// Forward / backward of the linear layer.  `ws` is device scratch sized by the
// matching *_workspace_bytes function below.
struct LinearArgs {
  int64_t T, K, N;
  int32_t r;
  float s;  // alpha / r
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;  // [K,r]
  const uint16_t* B;  // [r,N]
};

size_t fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r);
size_t bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r);

hipError_t launch_linear_fwd(const LinearArgs& a, const Codebook& cb, const uint16_t* X, uint16_t* Y, float* XA,
                             void* ws, hipStream_t s);
hipError_t launch_linear_bwd(const LinearArgs& a, const Codebook& cb, const uint16_t* dY, const uint16_t* X,
                             const float* XA, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, hipStream_t s);

}  // namespace qlora
