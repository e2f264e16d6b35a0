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
// on timing; the linear's first workgroup also returns it.
//
// Both kernels serve a group of up to kGemvGroupMax linears in one launch
// (the grouped small-token path: q/k/v, gate/up, or every linear of a
// layer at once): each linear owns a contiguous range of workgroups, so the
// launch and ramp are paid once for the whole group and the weight streams
// of all its linears overlap.  A single linear is a group of one.
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"

namespace qlora {

namespace {
constexpr int kRowsPerWG = 16;
constexpr int kWaves = 8;  // of the GEMV; the XA partial kernel has 8 too
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxR = 128;
constexpr int kAWinBytes = 65536;  // A window of an XA workgroup in LDS
constexpr int kXWin = 512;         // widest k window (RP = 64)
constexpr int kXPitch = kXWin + 8; // bf16 per staged X row
constexpr int kMaxParts = 32;           // XA partial slices per linear
constexpr int kPartLdsBytes = 36864;    // LDS area of the XA partials / the wave sums
constexpr int kXaPitch = kMaxR + 4;  // floats per row of XA / B^T in LDS (16-byte rows)
}  // namespace

// XA partial of slice b = blockIdx.x: P[b][t][j] = sum over k in
// [b ks, min(K, (b+1) ks)) of X[t][k] A[k][j], for t < 16 (rows t >= T are
// not stored) and j < RP (zero past r).  XA^T tiles (16 columns of A x 16
// token columns) are 16x16x32 MFMAs: wave w takes tile w % (RP/16) and every
// (8 / (RP/16))-th 32-k step of each window, starting at w / (RP/16).  A
// window's rows of A are contiguous, so they are staged with plain 16-byte
// loads and read back column-wise from LDS.
template <int NMAX>
__global__ __launch_bounds__(512) void xa_partial_kernel(GemvGroupT<NMAX> G) {
  // The linear of this workgroup (uniform: a scalar search over the group).
  int li = 0;
#pragma unroll
  for (int j = 1; j < NMAX; ++j)
    if (j < G.count && (int)blockIdx.x >= G.L[j].part_begin) li = j;
  const GemvLinear& Lin = G.L[li];
  const uint16_t* __restrict__ X = Lin.X;
  const uint16_t* __restrict__ A = Lin.A;
  float* __restrict__ P = Lin.P;
  const int T = G.T, r = G.r, RP = G.RP, ks = Lin.ks;
  const int64_t K = Lin.K;
  const int pb = (int)blockIdx.x - Lin.part_begin;  // slice of this linear
  __shared__ __align__(16) uint16_t as_[kAWinBytes / 2];
  __shared__ __align__(16) uint16_t xs_[16 * kXPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int kw = kAWinBytes / 2 / RP;  // 512 (RP = 64) or 256 (RP = 128)
  const int64_t kb0 = (int64_t)pb * ks;
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
    P[(int64_t)pb * nvals + v] = sum;
  }
}

// Registers of one 128-k chunk of a wave: RG row groups of 16 rows share
// one set of X operands.
template <int RG>
struct ChunkRegs {
  u32x4 c[RG];     // 32 codes of this lane's row in each row group
  uint32_t q[RG];  // q8 of the lane's block in each row group
  float s2[RG];    // s2 of those blocks' groups
  u32x4 x[4];      // X[t][k0 + 8s .. +8], s = 0..3
};

// RG: row groups of 16 rows per workgroup (and per wave chunk).  More row
// groups put more weight bytes in flight per wave (4 KiB per chunk at
// RG = 4) and share each X load among more rows; the launcher picks RG so
// the grid still fills the GPU.
template <int RG, int NMAX>
__global__ __launch_bounds__(kThreads) void gemv_fwd_kernel(GemvGroupT<NMAX> G, Codebook cb) {
  constexpr int ROWS = 16 * RG;
  static_assert(kWaves * ROWS * 17 * 4 <= kPartLdsBytes, "wave sums fit the partial area");
  int li = 0;
#pragma unroll
  for (int j = 1; j < NMAX; ++j)
    if (j < G.count && (int)blockIdx.x >= G.L[j].wg_begin) li = j;
  const GemvLinear& p = G.L[li];
  const int bid = (int)blockIdx.x - p.wg_begin;  // workgroup of this linear
  __shared__ __align__(4096) unsigned char tbl[2048];    // codebook pair table at LDS address 0
  // XA partials [nparts][T][RP] (copied in at the start); after they are
  // summed, the waves' partial outputs [kWaves][ROWS][17].
  __shared__ __align__(16) float ps[kPartLdsBytes / 4];
  __shared__ __align__(16) float xa_s[16][kXaPitch];       // XA[t][j]
  __shared__ __align__(16) uint16_t b_s[kMaxR * ROWS];     // B[j][n0 + nn] at j * ROWS + nn

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t T = G.T, K = p.K, N = p.N;
  const int r = G.r, RP = G.RP;
  const int64_t n0 = (int64_t)bid * ROWS;
  const int64_t K2 = K / 2, bpr = K / 64;

  const int64_t nchunk = (K + 127) / 128;
  const rsrc_t rc = make_rsrc(p.codes, N * K2);
  const rsrc_t rq = make_rsrc(p.q8, N * bpr);
  const rsrc_t rs = make_rsrc(p.s2, ((N * bpr + 255) / 256) * 4);
  const rsrc_t rx = make_rsrc(p.X, T * K * 2);
  // This wave's chunks are c = wave + 8 m, m < nmine.
  const int nmine = nchunk > wave ? (int)((nchunk - wave + kWaves - 1) / kWaves) : 0;
  // Unconditional buffer loads (reads past a view's end return zero): rows
  // n >= N read zero codes and scales; a 32-k group past K, and every load
  // of a chunk m >= nmine, has its offset pushed out of range, so it reads
  // zero without memory traffic.  With no branch around the loads, the
  // compiler counts the loads in flight exactly and waits only for the
  // chunk it is about to use.
  auto load = [&](int m, ChunkRegs<RG>& R) {
    const int64_t k0 = (int64_t)(wave + kWaves * m) * 128 + 32 * g;
    const bool kv = m < nmine && k0 < K;  // K % 64 == 0: a 32-k group is whole or absent
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int64_t n = n0 + 16 * rg + l16;
      R.c[rg] = buf_load16(rc, off_if(kv, (uint32_t)(n * K2 + k0 / 2)));
      const int64_t b = n * bpr + k0 / 64;
      R.q[rg] = buf_load1(rq, off_if(kv, (uint32_t)b));
      R.s2[rg] = __uint_as_float(buf_load4(rs, off_if(kv, (uint32_t)((b >> 8) * 4))));
    }
    // Lanes of padding tokens (l16 >= T) read past the X view: zero, and no
    // memory traffic (an exec-masked load would cost more than this).
    const uint32_t xo = off_if(kv, (uint32_t)(((int64_t)l16 * K + k0) * 2));
#pragma unroll
    for (int s = 0; s < 4; ++s) R.x[s] = buf_load16(rx, xo + 16 * s);
  };

  // First the XA partials and the workgroup's B slice, copied straight into
  // LDS by buffer-to-LDS loads (no registers held; bytes past either view
  // read zero), then the codebook pair table, then the weight stream.
  const int nvals = (int)T * RP, nparts = p.nparts;
  {
    const rsrc_t rp = make_rsrc(p.P, (int64_t)nparts * nvals * 4);
    const int units = (nparts * nvals * 4 + 15) / 16;
    for (int u0 = wave * 64; u0 < units; u0 += kThreads)
      buf_load16_to_lds(rp, reinterpret_cast<unsigned char*>(ps) + u0 * 16, (uint32_t)((u0 + lane) * 16));
    // B row j, 16-byte unit cu of the workgroup's ROWS columns; rows j >= r
    // read zero.
    const rsrc_t rb = make_rsrc(p.B, (int64_t)r * N * 2);
    constexpr int kUnitsPerRow = ROWS / 8;
    for (int u0 = wave * 64; u0 < r * kUnitsPerRow; u0 += kThreads) {
      const int u = u0 + lane, j = u / kUnitsPerRow, cu = u % kUnitsPerRow;
      buf_load16_to_lds(rb, reinterpret_cast<unsigned char*>(b_s) + u0 * 16,
                        off_if(u < r * kUnitsPerRow, (uint32_t)(((int64_t)j * N + n0 + 8 * cu) * 2)));
    }
  }
  pair_table_from_arg(tbl, cb, tid);
  lds_barrier();  // the pair table (the copies above stay in flight)
  f32x4 acc[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
  ChunkRegs<RG> R[2];
  load(0, R[0]);
  load(1, R[1]);
  auto compute = [&](const ChunkRegs<RG>& C) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const float sc = dq_scale(C.q[rg], C.s2[rg]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float f[8];
        lut8_pairs(tbl, C.c[rg][s], f);
        acc[rg] = mfma16(as_bf16x8(pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                                   pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc)),
                         as_bf16x8(C.x[s]), acc[rg]);
      }
    }
  };
  // Pairs of chunks loop, the odd last chunk runs once after the loop, so
  // the back-edge is reached from one path and the wait counts stay exact:
  // each chunk waits only for its own loads, the next chunk's stay in
  // flight.
  int m = 0;
  for (; m + 2 <= nmine; m += 2) {
    compute(R[0]);
    load(m + 2, R[0]);
    compute(R[1]);
    load(m + 3, R[1]);
  }
  if (m < nmine) compute(R[0]);

  // XA = the partials added in slice order; the linear's first workgroup
  // also returns it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies into LDS
  __syncthreads();
  for (int v = tid; v < nvals; v += kThreads) {
    float x = ps[v];
    for (int b = 1; b < nparts; ++b) x += ps[b * nvals + v];
    const int t = v / RP, jj = v % RP;
    if (jj < r) {
      xa_s[t][jj] = x;
      if (bid == 0) p.XA[t * r + jj] = x;
    }
  }
  __syncthreads();  // the partials are consumed: their area takes the wave sums
  // D[n][t]: lane holds column t = l16 and rows 16 rg + 4g + i.
  float* const red = ps;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * ROWS + 16 * rg + 4 * g + i) * 17 + l16] = acc[rg][i];
  __syncthreads();

  for (int o = tid; o < (int)T * ROWS; o += kThreads) {
    const int t = o / ROWS, nn = o % ROWS;
    if (n0 + nn < N) {
      float y = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) y += red[(w * ROWS + nn) * 17 + t];
      // s XA[t] . B[:, n]: r % 8 == 0; two interleaved sums, added at the end.
      float lo0 = 0.0f, lo1 = 0.0f;
      for (int j = 0; j < r; j += 8) {
        const float4 a0 = *reinterpret_cast<const float4*>(&xa_s[t][j]);
        const float4 a1 = *reinterpret_cast<const float4*>(&xa_s[t][j + 4]);
        const uint16_t* bj = b_s + j * ROWS + nn;
        lo0 += a0.x * bf16_to_f32(bj[0 * ROWS]);
        lo1 += a0.y * bf16_to_f32(bj[1 * ROWS]);
        lo0 += a0.z * bf16_to_f32(bj[2 * ROWS]);
        lo1 += a0.w * bf16_to_f32(bj[3 * ROWS]);
        lo0 += a1.x * bf16_to_f32(bj[4 * ROWS]);
        lo1 += a1.y * bf16_to_f32(bj[5 * ROWS]);
        lo0 += a1.z * bf16_to_f32(bj[6 * ROWS]);
        lo1 += a1.w * bf16_to_f32(bj[7 * ROWS]);
      }
      const float lo = lo0 + lo1;
      y += G.s * lo;
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
  // the partials of all slices must fit the GEMV's LDS area
  int64_t cap = (int64_t)(kPartLdsBytes / 4) / (T * RP);
  if (cap > kMaxParts) cap = kMaxParts;
  if (np > cap) np = cap;
  if (np < 1) np = 1;
  const int64_t ks = ((K + np - 1) / np + 31) / 32 * 32;
  g.ks = (int)ks;
  g.nparts = (int)((K + ks - 1) / ks);  // every slice is non-empty
  return g;
}

namespace {
template <int NMAX>
hipError_t launch_gemv_kernels(const GemvGroupT<NMAX>& g, int parts, int wg, int RG, const Codebook& cb,
                               hipStream_t s) {
  {
    KernelTimer kt_("xa_partial_kernel", s);
    hipLaunchKernelGGL(xa_partial_kernel<NMAX>, dim3(parts), dim3(512), 0, s, g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("gemv_fwd_kernel", s);
    if (RG == 4) hipLaunchKernelGGL((gemv_fwd_kernel<4, NMAX>), dim3(wg), dim3(kThreads), 0, s, g, cb);
    else if (RG == 2) hipLaunchKernelGGL((gemv_fwd_kernel<2, NMAX>), dim3(wg), dim3(kThreads), 0, s, g, cb);
    else hipLaunchKernelGGL((gemv_fwd_kernel<1, NMAX>), dim3(wg), dim3(kThreads), 0, s, g, cb);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemv_group(GemvGroup g, const Codebook& cb, hipStream_t s) {
  // Linears with the longest rows first (a stable sort by K): their
  // workgroups take the longest, so starting them first keeps the last
  // round of the grid short.  Each linear keeps its own buffers, so the
  // order changes no result.
  for (int a = 1; a < g.count; ++a)
    for (int b = a; b > 0 && g.L[b].K > g.L[b - 1].K; --b) {
      const GemvLinear t = g.L[b];
      g.L[b] = g.L[b - 1];
      g.L[b - 1] = t;
    }
  // Row groups per workgroup: the most (4, 2, 1) that still gives at least
  // four workgroups per compute unit over the whole group.
  int RG = 4;
  for (; RG > 1; RG /= 2) {
    int64_t wgs = 0;
    for (int i = 0; i < g.count; ++i) wgs += (g.L[i].N + 16 * RG - 1) / (16 * RG);
    if (wgs >= 1024) break;
  }
  int wg = 0, parts = 0;
  for (int i = 0; i < g.count; ++i) {
    GemvLinear& L = g.L[i];
    const GemvPlan pl = gemv_plan(L.N, L.K, g.T, g.r);
    L.nparts = pl.nparts;
    L.ks = pl.ks;
    L.wg_begin = wg;
    L.part_begin = parts;
    wg += (int)((L.N + 16 * RG - 1) / (16 * RG));
    parts += pl.nparts;
  }
  if (g.count == 1) {
    GemvGroupT<1> g1{};
    g1.L[0] = g.L[0];
    g1.count = 1;
    g1.T = g.T;
    g1.r = g.r;
    g1.RP = g.RP;
    g1.s = g.s;
    return launch_gemv_kernels(g1, parts, wg, RG, cb, s);
  }
  return launch_gemv_kernels(g, parts, wg, RG, cb, s);
}

hipError_t launch_gemv_fwd(const FwdGemmParams& p, const Codebook& cb, hipStream_t s) {
  GemvGroup g{};
  g.count = 1;
  g.T = (int)p.T;
  g.r = p.r;
  g.RP = p.RP;
  g.s = p.s;
  GemvLinear& L = g.L[0];
  L.X = p.X;
  L.codes = p.codes;
  L.q8 = p.q8;
  L.s2 = p.s2;
  L.A = p.A;
  L.B = p.B;
  L.Y = p.Y;
  L.XA = p.XA;
  L.P = p.P;
  L.K = p.K;
  L.N = p.N;
  return launch_gemv_group(g, cb, s);
}

}  // namespace qlora
