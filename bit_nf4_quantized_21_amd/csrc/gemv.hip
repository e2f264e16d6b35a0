// Small-token forward (T <= 16): HBM-bound dequant-GEMV of the NF4 layer with
// the whole LoRA branch in the same launch, for gfx950.
//
//   XA = X A;   Y[t][n] = sum_k X[t][k] W'[n][k] + s sum_j XA[t][j] B[j][n]
//
// This is the shape of 4-bit inference and batched generation (QLoRA project
// page, inference features) where the 4-bit weight stream is the whole cost.
//
// Design: one workgroup = 8 waves = 16 rows of W.  Wave w takes the 128-k
// chunks w, w+8, w+16, ... of those rows, so every wave streams distinct code
// bytes and the 8 partial sums are reduced through LDS at the end.  Each lane
// owns one row and 32 consecutive k of a chunk (16 code bytes, one 16-byte
// load); the codes are decoded in registers straight into the A operand of a
// bf16 16x16x32 MFMA whose B operand is X padded to 16 token columns.  Each
// wave keeps two chunks in flight (the loads of chunk c + 16 are issued as
// soon as chunk c is decoded); deeper rings measured no faster at 4096 x
// 4096 and slower for larger N, where two workgroups share a compute unit.
//
// The adapter's down-projection XA = X A comes from a small kernel launched
// just before (xa_partial_kernel: workgroup b sums a slice of the
// contraction on MFMA and stores the fp32 partial).  The GEMV requests the
// partials right behind its first weight loads and adds them in slice order
// in its epilogue, so XA is the same in every workgroup and does not depend
// on timing; workgroup 0 also returns it.
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"

namespace qlora {

namespace {
constexpr int kRowsPerWG = 16;
constexpr int kWaves = 8;  // of the GEMV; the XA partial kernel has 8 too
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 2;    // chunks in flight per wave
constexpr int kMaxR = 128;
constexpr int kAWinBytes = 65536;  // A window of an XA workgroup in LDS
constexpr int kXWin = 512;         // widest k window (RP = 64)
constexpr int kXPitch = kXWin + 8; // bf16 per staged X row
constexpr int kPartRegs = 32;      // XA partial values one GEMV thread holds
constexpr int kXaPitch = kMaxR + 4;  // floats per row of XA / B^T in LDS (16-byte rows)
}  // namespace

// XA partial of slice b = blockIdx.x: P[b][t][j] = sum over k in
// [b ks, min(K, (b+1) ks)) of X[t][k] A[k][j], for t < 16 (rows t >= T are
// not stored) and j < RP (zero past r).  XA^T tiles (16 columns of A x 16
// token columns) are 16x16x32 MFMAs: wave w takes tile w % (RP/16) and every
// (8 / (RP/16))-th 32-k step of each window, starting at w / (RP/16).  A
// window's rows of A are contiguous, so they are staged with plain 16-byte
// loads and read back column-wise from LDS.
__global__ __launch_bounds__(512) void xa_partial_kernel(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ A, float* __restrict__ P,
                                                         int T, int64_t K, int r, int RP, int ks) {
  __shared__ __align__(16) uint16_t as_[kAWinBytes / 2];
  __shared__ __align__(16) uint16_t xs_[16 * kXPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int kw = kAWinBytes / 2 / RP;  // 512 (RP = 64) or 256 (RP = 128)
  const int64_t kb0 = (int64_t)blockIdx.x * ks;
  const int64_t kb1 = kb0 + ks < K ? kb0 + ks : K;
  const rsrc_t ra = make_rsrc(A, K * r * 2);
  const rsrc_t rx = make_rsrc(X, (int64_t)T * K * 2);
  const int ntile = RP / 16, wpt = 8 / ntile;
  const int jt = wave % ntile, wk = wave / ntile;
  const int j = jt * 16 + l16;
  f32x4 xd = {0.f, 0.f, 0.f, 0.f};
  for (int64_t w0 = kb0; w0 < kb1; w0 += kw) {
    const int nk = kb1 - w0 < kw ? (int)(kb1 - w0) : kw;  // a multiple of 32
    const uint32_t abytes = (uint32_t)(nk * r * 2);
    u32x4 pa[8], px[2];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t off = (uint32_t)(tid + 512 * q) * 16;
      pa[q] = buf_load16(ra, off_if(off < abytes, (uint32_t)(w0 * r * 2) + off));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 512 * q, t = e >> 6, kk = (e & 63) * 8;  // X row t, k = w0 + kk
      px[q] = buf_load16(rx, off_if(t < T && kk < nk, (uint32_t)((t * K + w0 + kk) * 2)));
    }
    if (w0 != kb0) __syncthreads();  // the previous window is consumed
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4*>(&as_[(tid + 512 * q) * 8]) = pa[q];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 512 * q;
      *reinterpret_cast<u32x4*>(&xs_[(e >> 6) * kXPitch + (e & 63) * 8]) = px[q];
    }
    __syncthreads();
    for (int st = wk; st < nk / 32; st += wpt) {
      const int kk = st * 32 + 8 * g;
      uint32_t a2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = j < r ? as_[(kk + 2 * e) * r + j] : 0u;
        const uint32_t hi = j < r ? as_[(kk + 2 * e + 1) * r + j] : 0u;
        a2[e] = lo | (hi << 16);
      }
      const u32x4 xo = *reinterpret_cast<const u32x4*>(&xs_[l16 * kXPitch + kk]);
      xd = mfma16(as_bf16x8(a2[0], a2[1], a2[2], a2[3]), as_bf16x8(xo), xd);
    }
  }
  __syncthreads();
  // D[j][t]: lane holds t = l16 and j = jt*16 + 4g + i.  The waves' k-phases
  // are added in order through LDS (over the A window).
  float* const xt = reinterpret_cast<float*>(as_);  // [wpt][RP][17]
#pragma unroll
  for (int i = 0; i < 4; ++i) xt[(wk * RP + jt * 16 + 4 * g + i) * 17 + l16] = xd[i];
  __syncthreads();
  const int nvals = T * RP;
  for (int v = tid; v < nvals; v += 512) {
    const int t = v / RP, jj = v % RP;
    float sum = xt[jj * 17 + t];
    for (int h = 1; h < wpt; ++h) sum += xt[(h * RP + jj) * 17 + t];
    P[(int64_t)blockIdx.x * nvals + v] = sum;
  }
}

struct ChunkRegs {
  u32x4 c;      // 32 codes of this lane
  uint32_t q;   // q8 of the lane's block
  float s2;     // s2 of that block's group
  u32x4 x[4];   // X[t][k0 + 8s .. +8], s = 0..3
};

// NQ: XA values per thread (T * RP <= kThreads NQ); the thread holds all
// kPartRegs / NQ slices of each.
template <int NQ>
__global__ __launch_bounds__(kThreads) void gemv_fwd_kernel(FwdGemmParams p, Codebook cb) {
  constexpr int NP = kPartRegs / NQ;
  __shared__ __align__(4096) unsigned char tbl[2048];  // codebook pair table at LDS address 0
  __shared__ float red[kWaves][16][17];
  __shared__ __align__(16) float xa_s[16][kXaPitch];  // XA[t][j]
  __shared__ __align__(16) float bt_s[16][kXaPitch];  // B[j][n0 + nn] at [nn][j]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int r = p.r, RP = p.RP;
  const int64_t n0 = (int64_t)blockIdx.x * kRowsPerWG;
  const int64_t n = n0 + l16;
  const int64_t K2 = K / 2, bpr = K / 64;

  const int64_t nchunk = (K + 127) / 128;
  // Unconditional buffer loads (reads past a view's end return zero): rows
  // n >= N read zero codes and scales; a 32-k group past K reads some other
  // row's codes but a zero X (its offset is pushed out of range), so it adds
  // nothing.
  const rsrc_t rc = make_rsrc(p.codes, N * K2);
  const rsrc_t rq = make_rsrc(p.q8, N * bpr);
  const rsrc_t rs = make_rsrc(p.s2, ((N * bpr + 255) / 256) * 4);
  const rsrc_t rx = make_rsrc(p.X, T * K * 2);
  // Chunks past the last one are not requested (a branch uniform over the
  // wave): even a load that returns zero would take a slot in the memory
  // pipeline and hold its registers until it drains.
  auto load = [&](int64_t c, ChunkRegs& R) {
    if (c >= nchunk) return;
    const int64_t k0 = c * 128 + 32 * g;
    const bool kv = k0 < K;  // K % 64 == 0: a 32-k group is whole or absent
    R.c = buf_load16(rc, (uint32_t)(n * K2 + k0 / 2));
    const int64_t b = n * bpr + k0 / 64;
    R.q = buf_load1(rq, (uint32_t)b);
    R.s2 = __uint_as_float(buf_load4(rs, (uint32_t)((b >> 8) * 4)));
    // Lanes of padding tokens (l16 >= T) read past the X view: zero, and no
    // memory traffic (an exec-masked load would cost more than this).
    const uint32_t xo = off_if(kv, (uint32_t)(((int64_t)l16 * K + k0) * 2));
#pragma unroll
    for (int s = 0; s < 4; ++s) R.x[s] = buf_load16(rx, xo + 16 * s);
  };

  // The codebook pair table first (a barrier with no load outstanding costs
  // little), then the weight stream: four chunks of every wave in flight.
  pair_table_from_arg(tbl, cb, tid);
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ChunkRegs R[kRing] = {};
  const int64_t c0 = wave;
#pragma unroll
  for (int i = 0; i < kRing; ++i) load(c0 + i * kWaves, R[i]);

  // Then the XA partials this thread adds: part[q][b] is slice b of value
  // v = tid + kThreads q (slices past nparts read zero), and the workgroup's
  // r x 16 slice of B (value v = tid + kThreads q is B[v/16][n0 + v%16]).
  const int nvals = (int)T * RP, nparts = p.nparts;
  const rsrc_t rp = make_rsrc(p.P, (int64_t)nparts * nvals * 4);
  float part[NQ][NP];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int b = 0; b < NP; ++b) part[q][b] = 0.0f;
  if (wave * 64 < nvals) {  // waves whose first value is past the end hold none
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int v = tid + kThreads * q;
#pragma unroll
      for (int b = 0; b < NP; ++b)
        part[q][b] = __uint_as_float(buf_load4(rp, off_if(v < nvals && b < nparts, (uint32_t)((b * nvals + v) * 4))));
    }
  }
  const int nbv = r * kRowsPerWG;
  const rsrc_t rb = make_rsrc(p.B, (int64_t)r * N * 2);
  constexpr int kBq = kMaxR * kRowsPerWG / kThreads;
  uint32_t bv[kBq];
#pragma unroll
  for (int q = 0; q < kBq; ++q) {
    const int v = tid + kThreads * q;
    const int64_t nn = n0 + v % kRowsPerWG;
    bv[q] = buf_load2(rb, off_if(v < nbv && nn < N, (uint32_t)(((int64_t)(v / kRowsPerWG) * N + nn) * 2)));
  }
  for (int64_t cb0 = c0; cb0 < nchunk; cb0 += kRing * kWaves) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int64_t c = cb0 + i * kWaves;
      if (c >= nchunk) break;
      const float sc = dq_scale(R[i].q, R[i].s2);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float f[8];
        lut8_pairs(tbl, R[i].c[s], f);
        acc = mfma16(as_bf16x8(pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                               pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc)),
                     as_bf16x8(R[i].x[s]), acc);
      }
      load(c + kRing * kWaves, R[i]);
    }
  }
  // D[n][t]: lane holds column t = l16 and rows n = 4g + i.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][l16] = acc[i];
#pragma unroll
  for (int q = 0; q < kBq; ++q) {
    const int v = tid + kThreads * q;
    if (v < nbv) bt_s[v % kRowsPerWG][v / kRowsPerWG] = bf16_to_f32((uint16_t)bv[q]);
  }
  // XA = the partials added in slice order; workgroup 0 also returns it.
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int v = tid + kThreads * q;
    float x = part[q][0];
#pragma unroll
    for (int b = 1; b < NP; ++b) x += part[q][b];
    if (v < nvals) {
      const int t = v / RP, jj = v % RP;
      if (jj < r) {
        xa_s[t][jj] = x;
        if (blockIdx.x == 0) p.XA[t * r + jj] = x;
      }
    }
  }
  __syncthreads();

  if (tid < 256) {
    const int t = tid >> 4, nn = tid & 15;
    if (t < T && n0 + nn < N) {
      float y = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) y += red[w][nn][t];
      // s XA[t] . B[:, n]: r % 8 == 0; two interleaved sums, added at the end.
      float lo0 = 0.0f, lo1 = 0.0f;
      for (int j = 0; j < r; j += 8) {
        const float4 a0 = *reinterpret_cast<const float4*>(&xa_s[t][j]);
        const float4 a1 = *reinterpret_cast<const float4*>(&xa_s[t][j + 4]);
        const float4 b0 = *reinterpret_cast<const float4*>(&bt_s[nn][j]);
        const float4 b1 = *reinterpret_cast<const float4*>(&bt_s[nn][j + 4]);
        lo0 += a0.x * b0.x;
        lo1 += a0.y * b0.y;
        lo0 += a0.z * b0.z;
        lo1 += a0.w * b0.w;
        lo0 += a1.x * b1.x;
        lo1 += a1.y * b1.y;
        lo0 += a1.z * b1.z;
        lo1 += a1.w * b1.w;
      }
      const float lo = lo0 + lo1;
      y += p.s * lo;
      const uint32_t v = pack_bf16x2(y, 0.0f);
      p.Y[(int64_t)t * N + n0 + nn] = (uint16_t)(v & 0xFFFF);
    }
  }
}

GemvPlan gemv_plan(int64_t N, int64_t K, int64_t T, int32_t r) {
  GemvPlan g{};
  g.grid = (int)((N + kRowsPerWG - 1) / kRowsPerWG);
  const int64_t RP = (r + 63) / 64 * 64;
  int64_t np = (K + 127) / 128;  // slices of at least 128 k
  const int64_t nq = (T * RP + kThreads - 1) / kThreads;
  const int64_t cap = kPartRegs / (nq <= 1 ? 1 : nq <= 2 ? 2 : 4);
  if (np > cap) np = cap;
  if (np < 1) np = 1;
  const int64_t ks = ((K + np - 1) / np + 31) / 32 * 32;
  g.ks = (int)ks;
  g.nparts = (int)((K + ks - 1) / ks);  // every slice is non-empty
  return g;
}

hipError_t launch_gemv_fwd(const FwdGemmParams& p0, const Codebook& cb, hipStream_t s) {
  FwdGemmParams p = p0;
  const GemvPlan g = gemv_plan(p.N, p.K, p.T, p.r);
  p.nparts = g.nparts;
  {
    KernelTimer kt_("xa_partial_kernel", s);
    hipLaunchKernelGGL(xa_partial_kernel, dim3(g.nparts), dim3(512), 0, s, p.X, p.A, p.P, (int)p.T, p.K, p.r, p.RP,
                       g.ks);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("gemv_fwd_kernel", s);
    const int64_t nvals = p.T * p.RP;
    if (nvals <= kThreads) hipLaunchKernelGGL(gemv_fwd_kernel<1>, dim3(g.grid), dim3(kThreads), 0, s, p, cb);
    else if (nvals <= 2 * kThreads) hipLaunchKernelGGL(gemv_fwd_kernel<2>, dim3(g.grid), dim3(kThreads), 0, s, p, cb);
    else hipLaunchKernelGGL(gemv_fwd_kernel<4>, dim3(g.grid), dim3(kThreads), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
