// AdamW update of the LoRA adapters (QLoRA project page, technical
// architecture: AdamW and paged optimizers; challenges: gradient clipping for
// stability), for gfx950.
//
// The adapters of a model live in one flat buffer (views per linear), so one
// launch updates all of them:
//   g = c * grad,  m = b1 m + (1-b1) g,  v = b2 v + (1-b2) g^2,
//   p = p - lr (m / (1-b1^t) / (sqrt(v / (1-b2^t)) + eps) + wd p),
//   param = bf16(p)
// with c the global-norm clipping coefficient min(1, max / (|grad| + 1e-6)).
// The norm is summed in fp64 by a first kernel (fixed grid, one partial per
// workgroup) and every workgroup of the update adds the partials in the same
// fixed order, so the result is deterministic.  Master weights, m and v may
// live in device memory or in pinned host memory mapped into the GPU's
// address space (the paged mode: the optimizer state takes no HBM, and the
// update streams it over the host link).
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace qlora {

namespace {
constexpr int kOptThreads = 256;
constexpr int kNormParts = 1024;  // workgroups of the norm pass (fp64 partials)

__device__ __forceinline__ double block_sum(double x, double* red) {
#pragma unroll
  for (int off = 32; off; off >>= 1) x += __shfl_xor(x, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
}  // namespace

// partial[b] = sum of grad^2 over this workgroup's grid-stride elements (fp64).
__global__ __launch_bounds__(kOptThreads) void grad_sumsq_kernel(const uint16_t* __restrict__ grad, int64_t n,
                                                                 double* __restrict__ partial) {
  __shared__ double red[4];
  double acc = 0.0;
  const int64_t stride = (int64_t)gridDim.x * kOptThreads * 8;
  for (int64_t e = ((int64_t)blockIdx.x * kOptThreads + threadIdx.x) * 8; e < n; e += stride) {
    if (e + 8 <= n) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(grad + e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double a = (double)bf16_lo(u[q]), b = (double)bf16_hi(u[q]);
        acc += a * a;
        acc += b * b;
      }
    } else {
      for (int64_t i = e; i < n; ++i) {
        const double a = (double)bf16_to_f32(grad[i]);
        acc += a * a;
      }
    }
  }
  const double s = block_sum(acc, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

struct AdamwArgs {
  int64_t n;
  uint16_t* param;
  float* master;
  float* m;
  float* v;
  const uint16_t* grad;
  float b1, b2, eps, wd, lr;
  float step_size;      // lr / (1 - b1^t)
  float inv_sqrt_bc2;   // 1 / sqrt(1 - b2^t)
  float max_norm;       // <= 0: no clipping
  const double* partial;
  int nparts;
  float* norm_out;      // optional
};

__global__ __launch_bounds__(kOptThreads) void adamw_kernel(AdamwArgs a) {
  __shared__ double red[4];
  float c = 1.0f;
  if (a.nparts > 0) {
    // The global norm from the partials, in the same order in every
    // workgroup: thread t adds partials t, t + 256, ... then a fixed tree.
    double x = 0.0;
    for (int i = threadIdx.x; i < a.nparts; i += kOptThreads) x += a.partial[i];
    const double norm = sqrt(block_sum(x, red));
    const double cc = (double)a.max_norm / (norm + 1e-6);
    c = cc < 1.0 ? (float)cc : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.norm_out) *a.norm_out = (float)norm;
  }
  const float b1 = a.b1, b2 = a.b2, omb1 = 1.0f - a.b1, omb2 = 1.0f - a.b2;
  const int64_t stride = (int64_t)gridDim.x * kOptThreads * 8;
  for (int64_t e = ((int64_t)blockIdx.x * kOptThreads + threadIdx.x) * 8; e < a.n; e += stride) {
    const int cnt = a.n - e < 8 ? (int)(a.n - e) : 8;
    float g[8], p[8], mm[8], vv[8];
    if (cnt == 8) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(a.grad + e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        g[2 * q] = bf16_lo(u[q]);
        g[2 * q + 1] = bf16_hi(u[q]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 pm = *reinterpret_cast<const float4*>(a.master + e + 4 * h);
        const float4 m4 = *reinterpret_cast<const float4*>(a.m + e + 4 * h);
        const float4 v4 = *reinterpret_cast<const float4*>(a.v + e + 4 * h);
        p[4 * h] = pm.x; p[4 * h + 1] = pm.y; p[4 * h + 2] = pm.z; p[4 * h + 3] = pm.w;
        mm[4 * h] = m4.x; mm[4 * h + 1] = m4.y; mm[4 * h + 2] = m4.z; mm[4 * h + 3] = m4.w;
        vv[4 * h] = v4.x; vv[4 * h + 1] = v4.y; vv[4 * h + 2] = v4.z; vv[4 * h + 3] = v4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = i < cnt;
        g[i] = ok ? bf16_to_f32(a.grad[e + i]) : 0.0f;
        p[i] = ok ? a.master[e + i] : 0.0f;
        mm[i] = ok ? a.m[e + i] : 0.0f;
        vv[i] = ok ? a.v[e + i] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float gi = g[i] * c;
      mm[i] = b1 * mm[i] + omb1 * gi;
      vv[i] = b2 * vv[i] + omb2 * (gi * gi);
      const float denom = __fsqrt_rn(vv[i]) * a.inv_sqrt_bc2 + a.eps;
      p[i] = p[i] - (a.step_size * (mm[i] / denom) + a.lr * a.wd * p[i]);
    }
    if (cnt == 8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<float4*>(a.master + e + 4 * h) = make_float4(p[4 * h], p[4 * h + 1], p[4 * h + 2], p[4 * h + 3]);
        *reinterpret_cast<float4*>(a.m + e + 4 * h) = make_float4(mm[4 * h], mm[4 * h + 1], mm[4 * h + 2], mm[4 * h + 3]);
        *reinterpret_cast<float4*>(a.v + e + 4 * h) = make_float4(vv[4 * h], vv[4 * h + 1], vv[4 * h + 2], vv[4 * h + 3]);
      }
      *reinterpret_cast<u32x4*>(a.param + e) =
          u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    } else {
      for (int i = 0; i < cnt; ++i) {
        a.master[e + i] = p[i];
        a.m[e + i] = mm[i];
        a.v[e + i] = vv[i];
        a.param[e + i] = (uint16_t)(pack_bf16x2(p[i], 0.0f) & 0xFFFFu);
      }
    }
  }
}

size_t adamw_workspace_bytes(int64_t n) { return n > 0 ? kNormParts * sizeof(double) : 0; }

hipError_t launch_adamw(int64_t n, uint16_t* param, float* master, float* m, float* v, const uint16_t* grad,
                        int32_t step, float lr, float b1, float b2, float eps, float wd, float max_norm,
                        float* norm_out, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  AdamwArgs a{};
  a.n = n;
  a.param = param;
  a.master = master;
  a.m = m;
  a.v = v;
  a.grad = grad;
  a.b1 = b1;
  a.b2 = b2;
  a.eps = eps;
  a.wd = wd;
  a.lr = lr;
  const double bc1 = 1.0 - std::pow((double)b1, (double)step), bc2 = 1.0 - std::pow((double)b2, (double)step);
  a.step_size = (float)((double)lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.max_norm = max_norm;
  a.norm_out = norm_out;
  const bool clip = max_norm > 0.0f || norm_out != nullptr;
  if (clip) {
    a.partial = static_cast<const double*>(ws);
    a.nparts = kNormParts;
    KernelTimer kt_("grad_sumsq_kernel", s);
    hipLaunchKernelGGL(grad_sumsq_kernel, dim3(kNormParts), dim3(kOptThreads), 0, s, grad, n,
                       static_cast<double*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (max_norm <= 0.0f) a.max_norm = HUGE_VALF;  // norm reported, never clipped
  const int64_t per = (int64_t)kOptThreads * 8;
  int64_t grid = (n + per - 1) / per;
  if (grid > 8192) grid = 8192;
  {
    KernelTimer kt_("adamw_kernel", s);
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)grid), dim3(kOptThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace qlora
