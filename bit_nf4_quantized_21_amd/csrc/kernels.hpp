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
// Fused quantize + double quant (W fp32, or bf16 when `bf16`).
hipError_t launch_quantize_dq(const void* W, bool bf16, int64_t n, uint8_t* codes, uint8_t* q8, float* s2,
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
// True if every operand and workspace region of a T x K x N, rank-r problem
// fits the kernels' 32-bit buffer views.
bool linear_views_fit(int64_t T, int64_t K, int64_t N, int32_t r);
size_t bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r);

hipError_t launch_linear_fwd(const LinearArgs& a, const Codebook& cb, const uint16_t* X, uint16_t* Y, float* XA,
                             void* ws, hipStream_t s);
// One linear of a grouped forward (all share T, r and alpha).
struct GroupedLinear {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  float* XA;
  int64_t K, N;
};
size_t fwd_grouped_workspace_bytes(int count, const GroupedLinear* L, int64_t T, int32_t r);

// One linear of a grouped backward (all share T, r and alpha).
struct GroupedLinearBwd {
  const uint16_t* dY;
  const uint16_t* X;
  const float* XA;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* dX;
  uint16_t* dA;
  uint16_t* dB;
  int64_t K, N;
};
size_t bwd_grouped_workspace_bytes(int count, const GroupedLinearBwd* L, int64_t T, int32_t r);
hipError_t launch_linear_bwd_grouped(int count, const GroupedLinearBwd* L, int64_t T, int32_t r, float s,
                                     const Codebook& cb, void* ws, hipStream_t st);
hipError_t launch_linear_fwd_grouped(int count, const GroupedLinear* L, int64_t T, int32_t r, float s,
                                     const Codebook& cb, void* ws, hipStream_t st);

hipError_t launch_linear_bwd(const LinearArgs& a, const Codebook& cb, const uint16_t* dY, const uint16_t* X,
                             const float* XA, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, hipStream_t s);

// AdamW update of a flat adapter buffer (optim.hip); `ws` holds the fp64
// norm partials when clipping or the norm is asked for.
size_t adamw_workspace_bytes(int64_t n);
hipError_t launch_adamw(int64_t n, uint16_t* param, float* master, float* m, float* v, const uint16_t* grad,
                        int32_t step, float lr, float b1, float b2, float eps, float wd, float max_norm,
                        float* norm_out, void* ws, hipStream_t s);

}  // namespace qlora
