// Small-token forward (T <= 16): HBM-bound dequant-GEMV of the NF4 layer with
// the LoRA up-projection in the epilogue, for gfx950.
//
//   Y[t][n] = sum_k X[t][k] W'[n][k] + s sum_j XA[t][j] B[j][n]
//
// This is the shape of 4-bit inference and batched generation (QLoRA project
// page, inference features) where the 4-bit weight stream is the whole cost.
//
// Design: one workgroup = 8 waves = 16 rows of W.  Wave w takes the 128-k
// chunks w, w+8, w+16, ... of those rows, so every wave streams distinct code
// bytes and the 8 partial sums are reduced through LDS at the end.  Each lane
// owns one row and 32 consecutive k of a chunk (16 code bytes, one 16-byte
// load); the codes are decoded in registers straight into the A operand of a
// bf16 16x16x32 MFMA whose B operand is X padded to 16 token columns.  Loads
// are issued two chunks ahead of the decode so that a wave keeps ~8 KB of
// HBM traffic in flight.
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"

namespace qlora {

namespace {
constexpr int kRowsPerWG = 16;
constexpr int kWaves = 8;
constexpr int kMaxR = 128;
}  // namespace

struct ChunkRegs {
  u32x4 c;      // 32 codes of this lane
  uint32_t q;   // q8 of the lane's block
  float s2;     // s2 of that block's group
  u32x4 x[4];   // X[t][k0 + 8s .. +8], s = 0..3
};

__global__ __launch_bounds__(512) void gemv_fwd_kernel(FwdGemmParams p, Codebook cb) {
  __shared__ float lut[16];
  __shared__ float red[kWaves][16][17];
  __shared__ float xa_s[16][kMaxR + 1];
  __shared__ float b_s[kMaxR][17];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int r = p.r;
  const int64_t n0 = (int64_t)blockIdx.x * kRowsPerWG;
  const int64_t n = n0 + l16;
  const bool nval = n < N;
  const bool tval = l16 < T;
  const int64_t K2 = K / 2, bpr = K / 64;

  if (tid < 16) lut[tid] = cb.c[tid];
  for (int i = tid; i < (int)T * r; i += 512) xa_s[i / r][i % r] = p.XA[i];
  for (int i = tid; i < r * kRowsPerWG; i += 512) {
    const int j = i / kRowsPerWG, nn = i % kRowsPerWG;
    b_s[j][nn] = (n0 + nn < N) ? bf16_to_f32(p.B[(int64_t)j * N + n0 + nn]) : 0.0f;
  }
  __syncthreads();

  const int64_t nchunk = (K + 127) / 128;
  auto load = [&](int64_t c, ChunkRegs& R) {
    const int64_t k0 = c * 128 + 32 * g;
    const bool kv = k0 < K;  // K % 64 == 0: a 32-k group is whole or absent
    if (nval && kv) {
      R.c = *reinterpret_cast<const u32x4*>(p.codes + n * K2 + k0 / 2);
      const int64_t b = n * bpr + k0 / 64;
      R.q = p.q8[b];
      R.s2 = p.s2[b >> 8];
    } else {
      R.c = u32x4{0u, 0u, 0u, 0u};
      R.q = 0u;
      R.s2 = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      R.x[s] = (tval && kv) ? *reinterpret_cast<const u32x4*>(p.X + (int64_t)l16 * K + k0 + 8 * s)
                            : u32x4{0u, 0u, 0u, 0u};
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ChunkRegs R0 = {}, R1 = {}, R2 = {};
  int64_t c = wave;
  if (c < nchunk) load(c, R0);
  if (c + kWaves < nchunk) load(c + kWaves, R1);
  for (; c < nchunk; c += kWaves) {
    if (c + 2 * kWaves < nchunk) load(c + 2 * kWaves, R2);
    const float sc = dq_scale(R0.q, R0.s2);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t o[4];
      decode8_bf16(R0.c[s], sc, lut, o);
      acc = mfma16(as_bf16x8(o[0], o[1], o[2], o[3]), as_bf16x8(R0.x[s]), acc);
    }
    R0 = R1;
    R1 = R2;
  }
  // D[n][t]: lane holds column t = l16 and rows n = 4g + i.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][l16] = acc[i];
  __syncthreads();

  if (tid < 256) {
    const int t = tid >> 4, nn = tid & 15;
    if (t < T && n0 + nn < N) {
      float y = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) y += red[w][nn][t];
      float lo = 0.0f;
      for (int j = 0; j < r; ++j) lo += xa_s[t][j] * b_s[j][nn];
      y += p.s * lo;
      const uint32_t v = pack_bf16x2(y, 0.0f);
      p.Y[(int64_t)t * N + n0 + nn] = (uint16_t)(v & 0xFFFF);
    }
  }
}

hipError_t launch_gemv_fwd(const FwdGemmParams& p, const Codebook& cb, hipStream_t s) {
  const unsigned grid = (unsigned)((p.N + kRowsPerWG - 1) / kRowsPerWG);
  {
    KernelTimer kt_("gemv_fwd_kernel", s);
    hipLaunchKernelGGL(gemv_fwd_kernel, dim3(grid), dim3(512), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
