// Blockwise NF4 quantization, double quantization and dequantization kernels
// for gfx950.
//
// NF4 and double quantization are items (a) and (b) of the QLoRA abstract
// ("QLoRA: Efficient Finetuning of Quantized LLMs"); the block sizes (64 and
// 256), the 8-bit constant format and the low-nibble-first packing are the
// readings documented in include/qlora.h.
//
// All three kernels are HBM-bound streams.  The quantizer gives each 64-weight
// block to 16 lanes (one 16-byte load per lane, a 4-step shuffle max for the
// absmax), four blocks per lane group with their loads issued together, and
// decides every code exactly with fp64 products against the fp64 midpoints
// of the codebook; the double quantizer gives each group of 256
// constants to one wavefront.
#include <cmath>

#include "common.hpp"
#include "timing.hpp"
#include "kernels.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// Quantize: W[n] fp32 -> codes[n/2], absmax[ceil(n/64)].
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nf4_code(float w, double a64, const double* thr) {
  // code = #{j : w > absmax * m_j}; thr[j] = absmax * m_j is exact in fp64.
  double w64 = (double)w;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (w64 > thr[j]) ? 1u : 0u;
  return a64 == 0.0 ? 7u : c;
}

// Each 16-lane group quantizes kQGroupBlocks consecutive blocks; the loads of
// all of them are issued before any is used, so a wave keeps 4 KiB (fp32) or
// 2 KiB (bf16) of the weight stream in flight.  The per-weight decision work,
// not the bytes, bounds these kernels, so bf16 weights keep the same grid
// (8 blocks per group, half the waves, measured 13 % slower).
constexpr int kQGroupBlocks = 4;

// Four consecutive weights from e0 as fp32; zero past n.  A bf16 weight
// widens to fp32 exactly (its bits are the upper half of the fp32 word), so
// every decision below is the one taken for the same value given as fp32.
__device__ __forceinline__ void load_weights4(const float* __restrict__ W, int64_t n, int64_t e0, float (&v)[4]) {
  if (e0 + 4 <= n) {
    const float4 x = *reinterpret_cast<const float4*>(W + e0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < n) ? W[e0 + i] : 0.0f;
  }
}
__device__ __forceinline__ void load_weights4(const uint16_t* __restrict__ W, int64_t n, int64_t e0,
                                              float (&v)[4]) {
  if (e0 + 4 <= n) {
    const uint2 x = *reinterpret_cast<const uint2*>(W + e0);
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < n) ? __uint_as_float((uint32_t)W[e0 + i] << 16) : 0.0f;
  }
}
constexpr int kBins = 128;             // uniform bins of w / absmax over [-1, 1]
constexpr float kTinyAbsmax = 1e-30f;  // below this, blocks take the exact scan

// Nearest code by bins: every bin of width 2/kBins holds at most one decision
// boundary m_j, none within 1e-5 of a bin edge (checked on the host), so the
// bin of the fp32 estimate x = w * (1/absmax) (error < 1e-6) contains x's
// true position or is a neighbour separated from it by no boundary.  The code
// is the number of boundaries below the bin plus the exact fp64 decision
// w > absmax * m_j for the bin's own boundary (m = +inf when it has none).
template <typename T>
__device__ __forceinline__ void quantize_nf4_binned(const T* __restrict__ W, int64_t n, uint8_t* __restrict__ codes,
                                                    float* __restrict__ absmax, const Midpoints& mp) {
  __shared__ double s_thr[kBins];
  __shared__ uint32_t s_lo[kBins];
  if (threadIdx.x < kBins) {
    const double lo = -1.0 + threadIdx.x * (2.0 / kBins), hi = lo + 2.0 / kBins;
    uint32_t cnt = 0;
    double thr = __builtin_inf();
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      if (mp.m[j] < lo) cnt += 1;
      else if (mp.m[j] < hi) thr = mp.m[j];
    }
    s_thr[threadIdx.x] = thr;
    s_lo[threadIdx.x] = cnt;
  }
  __syncthreads();
  const int64_t nb = (n + kBlock - 1) / kBlock;
  constexpr int G = kQGroupBlocks;
  const int64_t blk0 = ((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) * G;
  const int l16 = threadIdx.x & 15;
  if (blk0 >= nb) return;  // whole 16-lane groups leave together (after the barrier)
  float v[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) load_weights4(W, n, (blk0 + g) * kBlock + l16 * 4, v[g]);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t blk = blk0 + g;
    if (blk >= nb) break;  // uniform per 16-lane group
    const int64_t e0 = blk * kBlock + l16 * 4;
    float a = fmaxf(fmaxf(fabsf(v[g][0]), fabsf(v[g][1])), fmaxf(fabsf(v[g][2]), fabsf(v[g][3])));
#pragma unroll
    for (int off = 8; off; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 16));
    if (l16 == 0) absmax[blk] = a;

    const double a64 = (double)a;
    uint32_t c[4];
    if (a < kTinyAbsmax) {  // uniform per 16-lane group; absmax 0 -> code 7
      double thr[15];
#pragma unroll
      for (int j = 0; j < 15; ++j) thr[j] = a64 * mp.m[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = nf4_code(v[g][i], a64, thr);
    } else {
      const float inv = __builtin_amdgcn_rcpf(a);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int b = (int)((v[g][i] * inv + 1.0f) * (0.5f * kBins));
        b = b < 0 ? 0 : (b > kBins - 1 ? kBins - 1 : b);
        c[i] = s_lo[b] + (((double)v[g][i] > a64 * s_thr[b]) ? 1u : 0u);
      }
    }
    const uint32_t packed = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12);
    if (blk * kBlock + kBlock <= n) {
      *reinterpret_cast<uint16_t*>(codes + e0 / 2) = (uint16_t)packed;
    } else {
      if (e0 < n) codes[e0 / 2] = (uint8_t)(packed & 0xFF);  // n is even: pairs are whole
      if (e0 + 2 < n) codes[e0 / 2 + 1] = (uint8_t)(packed >> 8);
    }
  }
}

// One kernel per weight type, so that traces tell them apart.
__global__ __launch_bounds__(256) void quantize_nf4_kernel(const float* __restrict__ W, int64_t n,
                                                           uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                           Midpoints mp) {
  quantize_nf4_binned(W, n, codes, absmax, mp);
}
__global__ __launch_bounds__(256) void quantize_nf4_bf16_kernel(const uint16_t* __restrict__ W, int64_t n,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ absmax, Midpoints mp) {
  quantize_nf4_binned(W, n, codes, absmax, mp);
}

// Exact linear scan over the 15 boundaries (used when the bins above do not
// separate the boundaries of the codebook in use).
template <typename T>
__global__ __launch_bounds__(256) void quantize_nf4_scan_kernel(const T* __restrict__ W, int64_t n,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax, Midpoints mp) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  constexpr int G = kQGroupBlocks;
  const int64_t blk0 = ((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) * G;
  const int l16 = threadIdx.x & 15;
  if (blk0 >= nb) return;  // whole 16-lane groups leave together
  float v[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) load_weights4(W, n, (blk0 + g) * kBlock + l16 * 4, v[g]);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t blk = blk0 + g;
    if (blk >= nb) break;  // uniform per 16-lane group
    const int64_t e0 = blk * kBlock + l16 * 4;
    float a = fmaxf(fmaxf(fabsf(v[g][0]), fabsf(v[g][1])), fmaxf(fabsf(v[g][2]), fabsf(v[g][3])));
#pragma unroll
    for (int off = 8; off; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 16));
    if (l16 == 0) absmax[blk] = a;

    const double a64 = (double)a;
    double thr[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) thr[j] = a64 * mp.m[j];
    const uint32_t c0 = nf4_code(v[g][0], a64, thr), c1 = nf4_code(v[g][1], a64, thr);
    const uint32_t c2 = nf4_code(v[g][2], a64, thr), c3 = nf4_code(v[g][3], a64, thr);
    const uint32_t packed = c0 | (c1 << 4) | (c2 << 8) | (c3 << 12);
    if (blk * kBlock + kBlock <= n) {
      *reinterpret_cast<uint16_t*>(codes + e0 / 2) = (uint16_t)packed;
    } else {
      if (e0 < n) codes[e0 / 2] = (uint8_t)(packed & 0xFF);  // n is even: pairs are whole
      if (e0 + 2 < n) codes[e0 / 2 + 1] = (uint8_t)(packed >> 8);
    }
  }
}

// ---------------------------------------------------------------------------
// Double quant: absmax[nb] -> q8[nb], s2[ceil(nb/256)].  One wave per group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t q8_code(float c, double s2d, double scale) {
  // Nearest integer to 255*c/s2, ties to even.  k0 = floor(c*255/s2) is
  // within one of the answer; 510*c and (2*k0+1)*s2 are exact in fp64 and
  // decide between k0 and k0+1.
  double cd = (double)c;
  double k0 = floor(cd * scale);
  double lhs = 510.0 * cd, rhs = (2.0 * k0 + 1.0) * s2d;
  int64_t k = (int64_t)k0;
  if (lhs > rhs || (lhs == rhs && (k & 1))) k += 1;
  k = k < 0 ? 0 : (k > 255 ? 255 : k);
  return (uint32_t)k;
}

__global__ __launch_bounds__(256) void double_quant_kernel(const float* __restrict__ absmax, int64_t nb,
                                                           uint8_t* __restrict__ q8, float* __restrict__ s2) {
  const int64_t ng = (nb + kBlock2 - 1) / kBlock2;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= ng) return;  // whole waves leave together
  const int64_t e0 = g * kBlock2 + lane * 4;
  const bool full = e0 + 4 <= nb;
  float v[4];
  if (full) {
    float4 x = *reinterpret_cast<const float4*>(absmax + e0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < nb) ? absmax[e0 + i] : 0.0f;
  }
  float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
  for (int off = 32; off; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) s2[g] = m;
  const double s2d = (double)m;
  const double scale = m > 0.0f ? 255.0 / s2d : 0.0;
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = m > 0.0f ? q8_code(v[i], s2d, scale) : 0u;
  if (full) {
    *reinterpret_cast<uint32_t*>(q8 + e0) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i < nb) q8[e0 + i] = (uint8_t)q[i];
  }
}

// ---------------------------------------------------------------------------
// Dequantize (support): 8 weights per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ q8,
                                                         const float* __restrict__ s2, int64_t n,
                                                         int out_bf16, void* __restrict__ out, Codebook cb) {
  __shared__ __align__(16) float lut[16];
  codebook_to_lds(lut, cb, threadIdx.x);
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= n) return;
  const int64_t b = e0 / kBlock;
  const float sc = dq_scale(q8[b], s2[b / kBlock2]);
  float w[8];
  if (e0 + 8 <= n) {
    uint32_t x = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = lut[(x >> (4 * i)) & 15] * sc;
    if (out_bf16) {
      u32x4 o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                 pack_bf16x2(w[6], w[7])};
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e0) = o;
    } else {
      float* o = reinterpret_cast<float*>(out) + e0;
      *reinterpret_cast<float4*>(o) = make_float4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(w[4], w[5], w[6], w[7]);
    }
  } else {
    for (int64_t e = e0; e < n; e += 2) {
      uint32_t x = codes[e / 2];
      float lo = lut[x & 15] * sc, hi = lut[x >> 4] * sc;
      if (out_bf16) {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + e) = pack_bf16x2(lo, hi);
      } else {
        reinterpret_cast<float*>(out)[e] = lo;
        reinterpret_cast<float*>(out)[e + 1] = hi;
      }
    }
  }
}

// ---------------------------------------------------------------------------
namespace {
template <typename T>
hipError_t launch_quantize_nf4_t(void (*binned_kernel)(const T*, int64_t, uint8_t*, float*, Midpoints),
                                 const T* W, int64_t n, uint8_t* codes, float* absmax, const Midpoints& mp,
                                 const char* name, hipStream_t s) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  constexpr int G = kQGroupBlocks;
  const int64_t grid = (nb + 16 * G - 1) / (16 * G);
  // The bins must hold at most one boundary each, none within 1e-5 of an edge.
  bool binned = true;
  for (int b = 0; b < kBins && binned; ++b) {
    const double lo = -1.0 + b * (2.0 / kBins), hi = lo + 2.0 / kBins;
    int inside = 0;
    for (int j = 0; j < 15; ++j) {
      if (mp.m[j] >= lo && mp.m[j] < hi) ++inside;
      if (std::fabs(mp.m[j] - lo) < 1e-5 || std::fabs(mp.m[j] - hi) < 1e-5) binned = false;
    }
    if (inside > 1) binned = false;
  }
  {
    KernelTimer kt_(name, s);
    if (binned)
      hipLaunchKernelGGL(binned_kernel, dim3((unsigned)grid), dim3(256), 0, s, W, n, codes, absmax, mp);
    else
      hipLaunchKernelGGL(quantize_nf4_scan_kernel<T>, dim3((unsigned)grid), dim3(256), 0, s, W, n, codes, absmax,
                         mp);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize_nf4(const float* W, int64_t n, uint8_t* codes, float* absmax, const Midpoints& mp,
                               hipStream_t s) {
  return launch_quantize_nf4_t(quantize_nf4_kernel, W, n, codes, absmax, mp, "quantize_nf4_kernel", s);
}

hipError_t launch_quantize_nf4_bf16(const uint16_t* W, int64_t n, uint8_t* codes, float* absmax,
                                    const Midpoints& mp, hipStream_t s) {
  return launch_quantize_nf4_t(quantize_nf4_bf16_kernel, W, n, codes, absmax, mp, "quantize_nf4_bf16_kernel",
                               s);
}

hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* q8, float* s2, hipStream_t s) {
  const int64_t ng = (nb + kBlock2 - 1) / kBlock2;
  const int64_t grid = (ng + 3) / 4;
  {
    KernelTimer kt_("double_quant_kernel", s);
    hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, absmax, nb, q8, s2);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                             int out_bf16, void* out, const Codebook& cb, hipStream_t s) {
  const int64_t groups = (n + 7) / 8;
  const int64_t grid = (groups + 255) / 256;
  {
    KernelTimer kt_("dequantize_kernel", s);
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, q8, s2, n, out_bf16,
                     out, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
