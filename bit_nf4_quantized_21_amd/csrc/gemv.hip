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
// are issued four chunks ahead of the decode, the first four before the
// workgroup's other set-up, so a wave keeps ~16 KB of traffic in flight.
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
  __shared__ __align__(16) float lut[16];
  __shared__ float red[kWaves][16][17];
  __shared__ float xa_s[16][kMaxR + 1];
  __shared__ float b_s[kMaxR][17];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int r = p.r;
  const int64_t n0 = (int64_t)blockIdx.x * kRowsPerWG;
  const int64_t n = n0 + l16;
  const int64_t K2 = K / 2, bpr = K / 64;

  const int64_t nchunk = (K + 127) / 128;
  // Unconditional buffer loads (reads past a view's end return zero): rows
  // n >= N read zero codes and scales; a 32-k group past K reads some other
  // row's codes but a zero X (its offset is pushed out of range), so it adds
  // nothing.  Chunks past the last are loaded and never used.
  const rsrc_t rc = make_rsrc(p.codes, N * K2);
  const rsrc_t rq = make_rsrc(p.q8, N * bpr);
  const rsrc_t rs = make_rsrc(p.s2, ((N * bpr + 255) / 256) * 4);
  const rsrc_t rx = make_rsrc(p.X, T * K * 2);
  // A chunk past the last one loads nothing at all: its offsets are pushed
  // past every view (no memory traffic, no branch).
  auto load = [&](int64_t c, ChunkRegs& R) {
    const int64_t k0 = c * 128 + 32 * g;
    const bool cv = c < nchunk;
    const bool kv = k0 < K;  // K % 64 == 0: a 32-k group is whole or absent
    R.c = buf_load16(rc, off_if(cv, (uint32_t)(n * K2 + k0 / 2)));
    const int64_t b = n * bpr + k0 / 64;
    R.q = buf_load1(rq, off_if(cv, (uint32_t)b));
    R.s2 = __uint_as_float(buf_load4(rs, off_if(cv, (uint32_t)((b >> 8) * 4))));
    const uint32_t xo = off_if(kv, (uint32_t)(((int64_t)l16 * K + k0) * 2));
#pragma unroll
    for (int s = 0; s < 4; ++s) R.x[s] = buf_load16(rx, xo + 16 * s);
  };

  // The adapter operands are requested first: the rowdot's chunk partials of
  // XA (T*RP <= 2048 values, at most 8 chunks each; value v = tid + 512q)
  // and the workgroup's r x 16 slice of B, from clamped in-bounds addresses
  // or zero-returning offsets; then the first four weight chunks of every
  // wave.  The adapter values are summed and stored to LDS once they arrive,
  // which waits for nothing issued after them.
  const int RPv = p.RP, nv = (int)T * RPv, nbv = r * kRowsPerWG;
  const rsrc_t rp = make_rsrc(p.P, (int64_t)p.nc * nv * 4);
  float xpart[4][8];
  uint16_t bv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = tid + 512 * q;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      xpart[q][c] = __uint_as_float(buf_load4(rp, off_if(v < nv && c < p.nc, (uint32_t)((c * nv + v) * 4))));
    const int ib = v < nbv ? v : nbv - 1;
    const int64_t nn = n0 + ib % kRowsPerWG;
    bv[q] = p.B[(int64_t)(ib / kRowsPerWG) * N + (nn < N ? nn : N - 1)];
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ChunkRegs R[4] = {};
  const int64_t c0 = wave;
#pragma unroll
  for (int i = 0; i < 4; ++i) load(c0 + i * kWaves, R[i]);

  codebook_to_lds(lut, cb, tid);
  // XA = the chunk partials summed in chunk order; workgroup 0 also returns it.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = tid + 512 * q;
    float x = xpart[q][0];
#pragma unroll
    for (int c = 1; c < 8; ++c) x += xpart[q][c];  // chunks past nc read zero
    if (v < nv) {
      const int t = v / RPv, j = v % RPv;
      if (j < r) {
        xa_s[t][j] = x;
        if (blockIdx.x == 0) p.XA[t * r + j] = x;
      }
    }
    if (v < nbv) b_s[v / kRowsPerWG][v % kRowsPerWG] = n0 + v % kRowsPerWG < N ? bf16_to_f32(bv[q]) : 0.0f;
  }
  __syncthreads();

  for (int64_t cb0 = c0; cb0 < nchunk; cb0 += 4 * kWaves) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t c = cb0 + i * kWaves;
      if (c >= nchunk) break;
      const float sc = dq_scale(R[i].q, R[i].s2);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        decode8_bf16(R[i].c[s], sc, lut, o);
        acc = mfma16(as_bf16x8(o[0], o[1], o[2], o[3]), as_bf16x8(R[i].x[s]), acc);
      }
      load(c + 4 * kWaves, R[i]);
    }
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
