// Skinny rank-r GEMMs of the LoRA adapter for gfx950 (LoRA tutorial,
// weight-update section: dW = W_A W_B; QLoRA abstract: gradients flow into
// the adapters only).
//
//   rowdot:  P[c][t][j] = sum_{l in chunk c} M[t][l] V(j,l)      (XA = X A,  G = dY B^T)
//   tokdot:  P[c][m][j] = sum_{t in chunk c} M[t][m] S[t][j]      (dA ~ X^T G, dB^T ~ dY^T XA)
// followed by fixed-order reductions of the chunk partials (deterministic,
// no float atomics).  All are HBM-bound streams over X or dY; the products
// run on bf16 MFMA 16x16x32 with fp32 accumulation.  The fp32 factors S (XA
// and G) enter the MFMA as a bf16 hi + lo pair, which keeps the adapter
// gradients at ~16-bit operand precision.
#include "common.hpp"
#include "timing.hpp"
#include "lora.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// rowdot.  One workgroup = 4 waves = 64 rows t of M; wave w owns rows
// [t0+16w, t0+16w+16) and every j.  MFMA orientation: D[j][t] (A = V^T, B = M).
// Lane (l16, g): A-operand row j = 16*jt + l16, B-operand column t = l16;
// both hold the 8 consecutive l = ks + 8g .. ks + 8g + 7.
// ---------------------------------------------------------------------------
template <bool VKMAJOR>
__global__ __launch_bounds__(256) void rowdot_partial_kernel(const uint16_t* __restrict__ M,
                                                             const uint16_t* __restrict__ V, float* __restrict__ P,
                                                             int64_t T, int64_t L, int r, int64_t LC) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t t = (int64_t)blockIdx.x * 64 + 16 * wave + l16;
  const int64_t c = blockIdx.y;
  const int64_t lbeg = c * LC;
  const int64_t lend = (lbeg + LC < L) ? lbeg + LC : L;
  const int njt = (r + 15) / 16;  // <= 8
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool tvalid = t < T;
  for (int64_t ks = lbeg; ks < lend; ks += 32) {
    const int64_t l0 = ks + 8 * g;
    const bool lvalid = l0 < lend;  // L % 8 == 0: an 8-group is whole or absent
    u32x4 mv = {0u, 0u, 0u, 0u};
    if (tvalid && lvalid) mv = *reinterpret_cast<const u32x4*>(M + t * L + l0);
    const bf16x8 bop = as_bf16x8(mv);
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < njt) {
        const int j = 16 * jt + l16;
        u32x4 vv = {0u, 0u, 0u, 0u};
        if (j < r && lvalid) {
          if (VKMAJOR) {
            uint32_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = V[(l0 + i) * r + j];
            vv = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
          } else {
            vv = *reinterpret_cast<const u32x4*>(V + (int64_t)j * L + l0);
          }
        }
        acc[jt] = mfma16(as_bf16x8(vv), bop, acc[jt]);
      }
    }
  }
  if (!tvalid) return;
  // D[j][t]: this lane holds column t and rows j = 16*jt + 4g + i.
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    const int j = 16 * jt + 4 * g;
    if (jt < njt && j < r) {
      float4 o = make_float4(acc[jt][0], acc[jt][1], acc[jt][2], acc[jt][3]);
      *reinterpret_cast<float4*>(P + (c * T + t) * r + j) = o;
    }
  }
}

// out[t][j] = sum_c P[c][t][j], fixed order.  One thread per 4 outputs.
__global__ __launch_bounds__(256) void rowdot_reduce_kernel(const float* __restrict__ P, float* __restrict__ out,
                                                            int64_t T, int r, int nc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total4 = T * r / 4;
  if (q >= total4) return;
  float4 s = *reinterpret_cast<const float4*>(P + 4 * q);
  for (int c = 1; c < nc; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(P + (int64_t)c * T * r + 4 * q);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(out + 4 * q) = s;
}

// ---------------------------------------------------------------------------
// tokdot.  One workgroup = 4 waves = 64 columns m of M; wave w owns columns
// [m0+16w, m0+16w+16).  MFMA orientation: D[j][m] (A = S^T as hi+lo, B = M).
// Lane (l16, g) holds tokens t = ts + 8g .. ts + 8g + 7 of its row / column.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tokdot_partial_kernel(const uint16_t* __restrict__ M,
                                                             const float* __restrict__ S, float* __restrict__ P,
                                                             int64_t T, int64_t C, int r, int64_t TC) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t m = (int64_t)blockIdx.x * 64 + 16 * wave + l16;
  const int64_t c = blockIdx.y;
  const int64_t tbeg = c * TC;
  const int64_t tend = (tbeg + TC < T) ? tbeg + TC : T;
  const int njt = (r + 15) / 16;
  const bool mvalid = m < C;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t ts = tbeg; ts < tend; ts += 32) {
    const int64_t t0 = ts + 8 * g;
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (mvalid && t0 + i < tend) ? M[(t0 + i) * C + m] : 0u;
    const bf16x8 bop =
        as_bf16x8(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < njt) {
        const int j = 16 * jt + l16;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (j < r && t0 + i < tend) ? S[(t0 + i) * r + j] : 0.0f;
        bf16x8 hi, lo;
        split_bf16x8(v, hi, lo);
        acc[jt] = mfma16(hi, bop, acc[jt]);
        acc[jt] = mfma16(lo, bop, acc[jt]);
      }
    }
  }
  if (!mvalid) return;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    const int j = 16 * jt + 4 * g;
    if (jt < njt && j < r) {
      float4 o = make_float4(acc[jt][0], acc[jt][1], acc[jt][2], acc[jt][3]);
      *reinterpret_cast<float4*>(P + (c * C + m) * r + j) = o;
    }
  }
}

// out = bf16(s * sum_c P[c][m][j]); layout [m][j] (dA: [K,r]) or [j][m]
// (dB: [r,N]).  One thread per 4 consecutive j.
__global__ __launch_bounds__(256) void tokdot_reduce_kernel(const float* __restrict__ P, uint16_t* __restrict__ out,
                                                            int64_t C, int r, int nc, float s, int transpose) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total4 = C * r / 4;
  if (q >= total4) return;
  float4 a = *reinterpret_cast<const float4*>(P + 4 * q);
  for (int c = 1; c < nc; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(P + (int64_t)c * C * r + 4 * q);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  const uint32_t p0 = pack_bf16x2(a.x * s, a.y * s), p1 = pack_bf16x2(a.z * s, a.w * s);
  const int64_t m = (4 * q) / r;
  const int j = (int)((4 * q) % r);
  if (!transpose) {
    *reinterpret_cast<uint2*>(out + 4 * q) = make_uint2(p0, p1);
  } else {
    out[(int64_t)(j + 0) * C + m] = (uint16_t)(p0 & 0xFFFF);
    out[(int64_t)(j + 1) * C + m] = (uint16_t)(p0 >> 16);
    out[(int64_t)(j + 2) * C + m] = (uint16_t)(p1 & 0xFFFF);
    out[(int64_t)(j + 3) * C + m] = (uint16_t)(p1 >> 16);
  }
}

// Zero-fill (used for dA / dB when there are no tokens).
__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_rowdot(const uint16_t* M, const uint16_t* V, bool v_kmajor, float* P, float* out, int64_t T,
                         int64_t L, int r, int64_t LC, hipStream_t s) {
  const int64_t nc = (L + LC - 1) / LC;
  dim3 grid((unsigned)((T + 63) / 64), (unsigned)nc);
  if (v_kmajor)
    {
      KernelTimer kt_("rowdot_partial_kernel", s);
      hipLaunchKernelGGL(rowdot_partial_kernel<true>, grid, dim3(256), 0, s, M, V, P, T, L, r, LC);
    }
  else
    {
      KernelTimer kt_("rowdot_partial_kernel", s);
      hipLaunchKernelGGL(rowdot_partial_kernel<false>, grid, dim3(256), 0, s, M, V, P, T, L, r, LC);
    }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("rowdot_reduce_kernel", s);
    hipLaunchKernelGGL(rowdot_reduce_kernel, dim3(blocks_for(T * r / 4)), dim3(256), 0, s, P, out, T, r, (int)nc);
  }
  return hipGetLastError();
}

hipError_t launch_tokdot(const uint16_t* M, const float* S, float* P, uint16_t* out, int64_t T, int64_t C, int r,
                         int64_t TC, float scale, bool transpose, hipStream_t s) {
  const int64_t nc = (T + TC - 1) / TC;
  dim3 grid((unsigned)((C + 63) / 64), (unsigned)nc);
  {
    KernelTimer kt_("tokdot_partial_kernel", s);
    hipLaunchKernelGGL(tokdot_partial_kernel, grid, dim3(256), 0, s, M, S, P, T, C, r, TC);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("tokdot_reduce_kernel", s);
    hipLaunchKernelGGL(tokdot_reduce_kernel, dim3(blocks_for(C * r / 4)), dim3(256), 0, s, P, out, C, r, (int)nc,
                     scale, transpose ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  {
    KernelTimer kt_("zero_u16_kernel", s);
    hipLaunchKernelGGL(zero_u16_kernel, dim3(blocks_for(n)), dim3(256), 0, s, p, n);
  }
  return hipGetLastError();
}

}  // namespace qlora
