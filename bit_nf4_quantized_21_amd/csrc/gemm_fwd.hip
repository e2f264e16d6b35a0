// Forward dequantize-GEMM of the frozen NF4 linear layer with the LoRA
// up-projection fused into its epilogue, for gfx950 (bf16 MFMA 32x32x16).
//
//   Y^T[n][m] = sum_k W'[n][k] X[m][k]  +  sum_j B[j][n] (s XA[m][j])
//
// W' = bf16(c[code] * fp32(q8*s2/255)) is the 4-bit base weight in the bf16
// compute dtype (QLoRA abstract items (a), (b); project page configuration
// example: NF4, double quantization, bf16 compute); the second term is the
// adapter's s (X A) B (LoRA tutorial, h = W x + dW x, with alpha/r scaling).
//
// Design (one workgroup = 4 waves = a 256 (n) x 256 (m) output tile):
//  * K advances one 64-weight quant block per step, so each W row contributes
//    exactly one 32-byte code segment and one scale per step.
//  * W' never touches LDS: lane (row, half) loads its 16 code bytes and
//    decodes them straight into the MFMA A-operand registers.  Each W row is
//    decoded once per workgroup (waves partition n), so the dequant cost is
//    amortised over 256 tokens.
//  * The contraction order inside a step is a fixed permutation of k: lane
//    half h, substep s, element i covers k = 32h + 8s + i.  X is read from
//    LDS in the same permuted order, so the sum is unchanged.
//  * X tiles (256 x 64 bf16) are double-buffered in LDS with a 144-byte row
//    pitch (16 consecutive rows hit 16 distinct 4-bank groups); the next
//    step's X and the step after next's codes are in flight during the MFMAs.
//  * Workgroup order is XCD-aware: tiles that share W rows are dispatched to
//    the same XCD so the codes are fetched from HBM once per L2.
#include "common.hpp"
#include "gemm.hpp"

namespace qlora {

namespace {
constexpr int kTileN = 256;
constexpr int kTileM = 256;
constexpr int kXPitch = 72;  // bf16 per LDS row (64 + 8)
}  // namespace

__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(FwdGemmParams p, Codebook cb) {
  __shared__ __align__(16) uint16_t xs[2][kTileM * kXPitch];
  __shared__ float lut[16];
  const int tid = threadIdx.x;

  const int bid = blockIdx.x;
  const int tile = (bid & 7) * p.per_xcd + (bid >> 3);
  if (tile >= p.tiles_n * p.tiles_m) return;  // uniform per workgroup, before any barrier
  const int tn = tile / p.tiles_m, tm = tile % p.tiles_m;

  if (tid < 16) lut[tid] = cb.c[tid];

  const int wave = tid >> 6, lane = tid & 63, ml = lane & 31, h = lane >> 5;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int64_t n0 = (int64_t)tn * kTileN, m0 = (int64_t)tm * kTileM;
  const int64_t K2 = K / 2, bpr = K / 64;
  const int nk = (int)(K / 64);

  int64_t nrow[2];
  bool nval[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    nrow[g] = n0 + 64 * wave + 32 * g + ml;
    nval[g] = nrow[g] < N;
  }
  const int xc = tid & 7, xr = tid >> 3;

  auto load_x = [&](int kb, u32x4(&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + xr + 32 * i;
      v[i] = (m < T) ? *reinterpret_cast<const u32x4*>(p.X + m * K + (int64_t)kb * 64 + xc * 8)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](int buf, const u32x4(&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&xs[buf][(xr + 32 * i) * kXPitch + xc * 8]) = v[i];
  };
  auto load_w = [&](int kb, u32x4(&c)[2], uint32_t(&q)[2], float(&sv)[2]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (nval[g]) {
        c[g] = *reinterpret_cast<const u32x4*>(p.codes + nrow[g] * K2 + (int64_t)kb * 32 + 16 * h);
        const int64_t b = nrow[g] * bpr + kb;
        q[g] = p.q8[b];
        sv[g] = p.s2[b >> 8];
      } else {
        c[g] = u32x4{0u, 0u, 0u, 0u};
        q[g] = 0u;
        sv[g] = 0.0f;
      }
    }
  };
  auto decode = [&](const u32x4(&c)[2], const uint32_t(&q)[2], const float(&sv)[2], bf16x8(&w)[2][4]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float sc = dq_scale(q[g], sv[g]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        decode8_bf16(c[g][s], sc, lut, o);
        w[g][s] = as_bf16x8(o[0], o[1], o[2], o[3]);
      }
    }
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[g][mi][e] = 0.0f;

  u32x4 xreg[8];
  u32x4 creg[2];
  uint32_t qreg[2];
  float sreg[2];
  bf16x8 wop[2][4];

  load_x(0, xreg);
  load_w(0, creg, qreg, sreg);
  __syncthreads();  // lut
  store_x(0, xreg);
  decode(creg, qreg, sreg, wop);
  if (nk > 1) load_w(1, creg, qreg, sreg);
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nk;
    if (more) load_x(kb + 1, xreg);
    u32x4 cn[2];
    uint32_t qn[2];
    float sn[2];
    if (kb + 2 < nk) load_w(kb + 2, cn, qn, sn);

    const uint16_t* xb = xs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 xop[8];
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        xop[mi] = *reinterpret_cast<const bf16x8*>(&xb[(32 * mi + ml) * kXPitch + 32 * h + 8 * s]);
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[g][mi] = mfma32(wop[g][s], xop[mi], acc[g][mi]);
    }
    if (more) {
      decode(creg, qreg, sreg, wop);
      store_x(buf ^ 1, xreg);
    }
    if (kb + 2 < nk) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        creg[g] = cn[g];
        qreg[g] = qn[g];
        sreg[g] = sn[g];
      }
    }
    __syncthreads();
  }

  // LoRA up-projection as one extra K-step of width r: A = B^T (rows n),
  // B operand = s * XA (columns m) as a bf16 hi + lo pair, so the fp32 XA
  // keeps ~16 significant bits even where the adapter term dominates Y.
  const int r = p.r;
  for (int c16 = 0; c16 < r; c16 += 16) {
    const int j0 = c16 + 8 * h;
    const bool jv = j0 < r;  // r % 8 == 0: the 8-group is whole or absent
    bf16x8 aop[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (nval[g] && jv) ? p.B[(int64_t)(j0 + i) * N + nrow[g]] : 0u;
      aop[g] = as_bf16x8(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      const int64_t m = m0 + 32 * mi + ml;
      float v[8];
      if (jv && m < T) {
        const float4 a = *reinterpret_cast<const float4*>(p.XA + m * r + j0);
        const float4 b = *reinterpret_cast<const float4*>(p.XA + m * r + j0 + 4);
        v[0] = a.x * p.s; v[1] = a.y * p.s; v[2] = a.z * p.s; v[3] = a.w * p.s;
        v[4] = b.x * p.s; v[5] = b.y * p.s; v[6] = b.z * p.s; v[7] = b.w * p.s;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      bf16x8 bhi, blo;
      split_bf16x8(v, bhi, blo);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        acc[g][mi] = mfma32(aop[g], bhi, acc[g][mi]);
        acc[g][mi] = mfma32(aop[g], blo, acc[g][mi]);
      }
    }
  }

  // D[n][m]: lane holds column m and rows n = 8*q4 + 4h + (0..3) of each 32x32 tile.
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    const int64_t m = m0 + 32 * mi + ml;
    if (m >= T) continue;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t n = n0 + 64 * wave + 32 * g + 8 * q4 + 4 * h;
        if (n < N) {
          const f32x16& a = acc[g][mi];
          uint2 o = make_uint2(pack_bf16x2(a[4 * q4 + 0], a[4 * q4 + 1]), pack_bf16x2(a[4 * q4 + 2], a[4 * q4 + 3]));
          *reinterpret_cast<uint2*>(p.Y + m * N + n) = o;
        }
      }
    }
  }
}

hipError_t launch_gemm_fwd(const FwdGemmParams& p0, const Codebook& cb, hipStream_t s) {
  FwdGemmParams p = p0;
  p.tiles_n = (int)((p.N + kTileN - 1) / kTileN);
  p.tiles_m = (int)((p.T + kTileM - 1) / kTileM);
  const int total = p.tiles_n * p.tiles_m;
  p.per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(gemm_fwd_kernel, dim3(8 * p.per_xcd), dim3(256), 0, s, p, cb);
  return hipGetLastError();
}

}  // namespace qlora
