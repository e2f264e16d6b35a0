// Backward dequantize-GEMM for the input gradient of the frozen NF4 layer,
// with the adapter's rank-r term fused into its epilogue, for gfx950.
//
//   dX^T[k][t] = sum_n W'[n][k] dY[t][n]  +  sum_j A[k][j] (s G[t][j])
//
// i.e. dX = dY W' + s G A^T with G = dY B^T: the gradient flowing through the
// frozen 4-bit weight and through the adapter (QLoRA abstract: backpropagation
// through the frozen 4-bit model into LoRA; the base weight gets no gradient).
//
// Design (one workgroup = 4 waves in a 2x2 grid = a 256 (k) x 256 (t) tile):
//  * The contraction runs over W's rows n, 64 per step.  The 64 x 256 block of
//    codes is loaded row-wise (coalesced), decoded once per workgroup and
//    written to LDS transposed ([k][n]) so the MFMA A operand reads 8
//    consecutive n with one 16-byte LDS load.  Each thread decodes an 8x8
//    patch (8 rows x 8 k) and writes 8 16-byte columns.
//  * dY tiles are staged in LDS in their natural [t][n] layout.
//  * LDS rows are 144 bytes and the 16-byte chunk index is XOR-swizzled with
//    bits 4..6 of the row, so both the transposed writes (rows 8 apart) and
//    the MFMA reads (16 consecutive rows) spread over distinct banks.
//  * Double-buffered: the next step's codes and dY are loaded during the
//    MFMAs of the current step and decoded / stored after them.
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"

namespace qlora {

namespace {
constexpr int kTileK = 256;
constexpr int kTileT = 256;
constexpr int kPitch = 72;  // bf16 per LDS row (64 + 8)

__device__ __forceinline__ int swz(int row, int chunk) { return row * kPitch + ((chunk ^ ((row >> 4) & 7)) << 3); }
}  // namespace

__global__ __launch_bounds__(256, 1) void gemm_dx_kernel(DxGemmParams p, Codebook cb) {
  __shared__ __align__(16) uint16_t wsm[2][kTileK * kPitch];
  __shared__ __align__(16) uint16_t dsm[2][kTileT * kPitch];
  __shared__ float lut[16];
  const int tid = threadIdx.x;

  const int bid = blockIdx.x;
  const int tile = (bid & 7) * p.per_xcd + (bid >> 3);
  if (tile >= p.tiles_k * p.tiles_t) return;  // uniform per workgroup, before any barrier
  const int tk = tile / p.tiles_t, tt = tile % p.tiles_t;
  if (tid < 16) lut[tid] = cb.c[tid];

  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wk = wave & 1, wt = wave >> 1;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int64_t k0 = (int64_t)tk * kTileK, t0 = (int64_t)tt * kTileT;
  const int64_t K2 = K / 2, bpr = K / 64;
  const int nsteps = (int)((N + 63) / 64);

  // dY loader: thread -> 16-byte chunk xc of rows xr + 32 i.
  const int xc = tid & 7, xr = tid >> 3;
  // Code loader: thread -> rows 8 rg .. 8 rg + 7 of the step, k = k0 + 8 kq .. + 7.
  const int rg = tid >> 5, kq = tid & 31;
  const int64_t kcol = k0 + 8 * kq;
  const bool kval = kcol < K;

  auto load_dy = [&](int st, u32x4(&v)[8]) {
    const int64_t nc = (int64_t)st * 64 + 8 * xc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = t0 + xr + 32 * i;
      v[i] = (t < T && nc < N) ? *reinterpret_cast<const u32x4*>(p.dY + t * N + nc) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_dy = [&](int buf, const u32x4(&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&dsm[buf][swz(xr + 32 * i, xc)]) = v[i];
  };
  auto load_w = [&](int st, uint32_t(&c)[8], uint32_t(&q)[8], float(&sv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = (int64_t)st * 64 + 8 * rg + i;
      if (n < N && kval) {
        c[i] = *reinterpret_cast<const uint32_t*>(p.codes + n * K2 + kcol / 2);
        const int64_t b = n * bpr + kcol / 64;
        q[i] = p.q8[b];
        sv[i] = p.s2[b >> 8];
      } else {
        c[i] = 0u;
        q[i] = 0u;
        sv[i] = 0.0f;
      }
    }
  };
  auto decode_store = [&](int buf, const uint32_t(&c)[8], const uint32_t(&q)[8], const float(&sv)[8]) {
    float v[8][8];  // [row i][k e]
#pragma unroll
    for (int i = 0; i < 8; ++i) decode8_f32(c[i], dq_scale(q[i], sv[i]), lut, v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4 o = {pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e]), pack_bf16x2(v[4][e], v[5][e]),
                 pack_bf16x2(v[6][e], v[7][e])};
      *reinterpret_cast<u32x4*>(&wsm[buf][swz(8 * kq + e, rg)]) = o;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  u32x4 dreg[8];
  uint32_t creg[8], qreg[8];
  float sreg[8];
  load_dy(0, dreg);
  load_w(0, creg, qreg, sreg);
  __syncthreads();  // lut
  decode_store(0, creg, qreg, sreg);
  store_dy(0, dreg);
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nsteps;
    if (more) {
      load_dy(st + 1, dreg);
      load_w(st + 1, creg, qreg, sreg);
    }
    const uint16_t* wb = wsm[buf];
    const uint16_t* db = dsm[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 aop[4], bop[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aop[i] = *reinterpret_cast<const bf16x8*>(&wb[swz(128 * wk + 32 * i + l32, 4 * h + s)]);
        bop[i] = *reinterpret_cast<const bf16x8*>(&db[swz(128 * wt + 32 * i + l32, 4 * h + s)]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(aop[a], bop[b], acc[a][b]);
    }
    if (more) {
      decode_store(buf ^ 1, creg, qreg, sreg);
      store_dy(buf ^ 1, dreg);
    }
    __syncthreads();
  }

  // Adapter term as one extra K-step of width r: A operand = A[k][j] (rows k),
  // B operand = s * G[t][j] (columns t) as a bf16 hi + lo pair.
  const int r = p.r;
  for (int c16 = 0; c16 < r; c16 += 16) {
    const int j0 = c16 + 8 * h;
    const bool jv = j0 < r;
    bf16x8 aop[4], bop[4], blo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = k0 + 128 * wk + 32 * i + l32;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (jv && k < K) v = *reinterpret_cast<const u32x4*>(p.A + k * r + j0);
      aop[i] = as_bf16x8(v);
      const int64_t t = t0 + 128 * wt + 32 * i + l32;
      float f[8];
      if (jv && t < T) {
        const float4 a = *reinterpret_cast<const float4*>(p.G + t * r + j0);
        const float4 b = *reinterpret_cast<const float4*>(p.G + t * r + j0 + 4);
        f[0] = a.x * p.s; f[1] = a.y * p.s; f[2] = a.z * p.s; f[3] = a.w * p.s;
        f[4] = b.x * p.s; f[5] = b.y * p.s; f[6] = b.z * p.s; f[7] = b.w * p.s;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.0f;
      }
      split_bf16x8(f, bop[i], blo[i]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[a][b] = mfma32(aop[a], bop[b], acc[a][b]);
        acc[a][b] = mfma32(aop[a], blo[b], acc[a][b]);
      }
  }

  // D[k][t]: lane holds column t and rows k = 8*q4 + 4h + (0..3) of each 32x32 tile.
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t t = t0 + 128 * wt + 32 * b + l32;
    if (t >= T) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t k = k0 + 128 * wk + 32 * a + 8 * q4 + 4 * h;
        if (k < K) {
          const f32x16& v = acc[a][b];
          uint2 o = make_uint2(pack_bf16x2(v[4 * q4 + 0], v[4 * q4 + 1]), pack_bf16x2(v[4 * q4 + 2], v[4 * q4 + 3]));
          *reinterpret_cast<uint2*>(p.dX + t * K + k) = o;
        }
      }
    }
  }
}

hipError_t launch_gemm_dx(const DxGemmParams& p0, const Codebook& cb, hipStream_t s) {
  DxGemmParams p = p0;
  p.tiles_k = (int)((p.K + kTileK - 1) / kTileK);
  p.tiles_t = (int)((p.T + kTileT - 1) / kTileT);
  const int total = p.tiles_k * p.tiles_t;
  p.per_xcd = (total + 7) / 8;
  {
    KernelTimer kt_("gemm_dx_kernel", s);
    hipLaunchKernelGGL(gemm_dx_kernel, dim3(8 * p.per_xcd), dim3(256), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
