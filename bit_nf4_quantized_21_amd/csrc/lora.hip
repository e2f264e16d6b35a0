// Skinny rank-r products of the LoRA adapter for gfx950 (LoRA tutorial,
// weight-update section: dW = W_A W_B with the alpha/r scale; QLoRA abstract:
// the frozen 4-bit base passes gradients into the adapters only).
//
//   rowdot:  out[t][j] = sum_l M[t][l] V(l, j)     XA = X A,   G = dY B^T
//   tokdot:  out[m][j] = s sum_t M[t][m] S[t][j]   dA = s X^T G,  dB^T = s dY^T XA
//
// Both stream a tall bf16 matrix M (X or dY) once from HBM; the rank-r
// factor is small and stays in L2.  Each is split into chunks of the
// contraction whose fp32 partials are summed in a fixed order by a second
// kernel, so results are bitwise reproducible (no float atomics).
//
// Products run on bf16 MFMA 16x16x32 with fp32 accumulation.  The MFMA wants
// 8 consecutive contraction indices per lane; where the contraction runs
// across rows of a row-major operand (A's rows in X A, the token rows of M in
// tokdot) each lane loads an 8 x 4 block and transposes it in registers with
// byte permutes, so lane p of an MFMA serves column 4p + c for c = 0..3 and
// the four MFMAs c together cover 64 columns.  The fp32 factors of tokdot
// (G, XA) enter as bf16 hi + lo planes written by the rowdot reduction.
#include "common.hpp"
#include "lora.hpp"
#include "timing.hpp"

namespace qlora {

namespace {

// Operand c (c = 0..3) of a lane's 8 x 4 bf16 block: rows i = 0..7 hold
// columns 4p .. 4p+3 as two dwords (cols 0,1 | cols 2,3); the operand packs
// column c of the 8 rows, row 2q in the low half of dword q.
__device__ __forceinline__ bf16x8 column_of(const uint2 (&rows)[8], int c) {
  const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = (c & 2) ? rows[2 * q].y : rows[2 * q].x;
    const uint32_t hi = (c & 2) ? rows[2 * q + 1].y : rows[2 * q + 1].x;
    d[q] = __builtin_amdgcn_perm(hi, lo, sel);
  }
  return as_bf16x8(d[0], d[1], d[2], d[3]);
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 buf_load_f4(rsrc_t r, uint32_t off) {
  const u32x4 u = buf_load16(r, off);
  return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3]));
}

}  // namespace

// ---------------------------------------------------------------------------
// rowdot partials.  Workgroup = 4 waves = 64 rows t of M x one chunk of l;
// wave w takes the w-th quarter of the chunk, 32 l per step.  MFMA
// orientation D[t][j]: A operand = M (row t = t0 + 16 tt + p, 8 consecutive
// l), B operand = V (8 consecutive l of column j = 64 jb + 4p + c).
// V_LR: V is stored [L][r] (the LoRA A); else [r][L] (the LoRA B).
// P[c][t][j] has row stride RP = 64 * JB.
// ---------------------------------------------------------------------------
template <bool V_LR, int JB>
__global__ __launch_bounds__(256) void rowdot_partial_kernel(RowdotJobs jobs, int64_t T, int64_t L, int r,
                                                             int64_t LC) {
  __shared__ __align__(16) float red[4][64 * 64];
  constexpr int RP = 64 * JB;
  // grid.y = jobs x chunks; the job of this workgroup is uniform
  const int job = __builtin_amdgcn_readfirstlane((int)blockIdx.y / jobs.nc);
  const uint16_t* __restrict__ M = jobs.M[job];
  const uint16_t* __restrict__ V = jobs.V[job];
  float* __restrict__ P = jobs.P[job];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, p = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int64_t ch = (int64_t)blockIdx.y - (int64_t)job * jobs.nc;
  const int64_t lbeg = ch * LC;
  const int64_t lend = lbeg + LC < L ? lbeg + LC : L;
  const int64_t LW = LC / 4;
  const int64_t wl0 = lbeg + wave * LW;
  const int64_t wl1 = wl0 + LW < lend ? wl0 + LW : lend;
  const int nsteps = wl1 > wl0 ? (int)((wl1 - wl0 + 31) / 32) : 0;

  f32x4 acc[JB][4][4];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[jb][tt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Regs {
    u32x4 m[4];
    u32x4 v[JB][4];   // V_LR == false: the operands themselves
    uint2 a[JB][8];   // V_LR: 8 rows x 4 columns per j-block, transposed at use
  };
  // Buffer views (this workgroup's rows of M; all of V): masked lanes load
  // zero through an offset past the view, so the loads carry no branches and
  // the next step's loads stay in flight while this step computes.
  const int64_t rows = T - t0 < 64 ? T - t0 : 64;
  const rsrc_t rm = make_rsrc(M + t0 * L, rows * L * 2);
  const rsrc_t rv = make_rsrc(V, (int64_t)r * L * 2);
  auto load = [&](int s, Regs& R) {
    const int64_t l = wl0 + 32 * s + 8 * g;
    const bool lv = l < wl1;  // L % 8 == 0: an 8-group is whole or absent
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      R.m[tt] = buf_load16(rm, off_if(lv, (uint32_t)(((16 * tt + p) * L + l) * 2)));
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      if constexpr (V_LR) {
        const int j = 64 * jb + 4 * p;
        const bool ok = lv && j < r;  // r % 8 == 0: a 4-group is whole or absent
#pragma unroll
        for (int i = 0; i < 8; ++i) R.a[jb][i] = buf_load8(rv, off_if(ok, (uint32_t)(((l + i) * r + j) * 2)));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 64 * jb + 4 * p + c;
          R.v[jb][c] = buf_load16(rv, off_if(lv && j < r, (uint32_t)((j * L + l) * 2)));
        }
      }
    }
  };
  auto compute = [&](const Regs& R) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 vop = V_LR ? column_of(R.a[jb], c) : as_bf16x8(R.v[jb][c]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[jb][tt][c] = mfma16(as_bf16x8(R.m[tt]), vop, acc[jb][tt][c]);
      }
    }
  };

  // Two register sets: the loads of step s+1 are in flight while step s runs.
  // A ring of D register sets: the loads of step s + D - 1 are issued
  // before step s computes, so D - 1 steps of loads are always in flight;
  // each slot is fenced so the compiler keeps that order.  Steps past the
  // wave's range load zeros.  (Deeper rings measured no faster: the
  // register cost lowers occupancy.)
  constexpr int D = 2;
  Regs R[D];
#pragma unroll
  for (int k = 0; k < D - 1; ++k) load(k, R[k]);
  for (int s = 0; s < nsteps; s += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load(s + k + D - 1, R[(k + D - 1) % D]);
      compute(R[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Sum the four waves' partials in wave order and store this chunk's tile.
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    if (jb) __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tt + 4 * g + i;
        *reinterpret_cast<float4*>(&red[wave][t * 64 + 4 * p]) =
            make_float4(acc[jb][tt][0][i], acc[jb][tt][1][i], acc[jb][tt][2][i], acc[jb][tt][3][i]);
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = threadIdx.x + 256 * k;
      const int t = q >> 4, j4 = q & 15;
      if (t0 + t >= T) continue;
      float4 sum = *reinterpret_cast<const float4*>(&red[0][t * 64 + 4 * j4]);
#pragma unroll
      for (int w = 1; w < 4; ++w) sum = add4(sum, *reinterpret_cast<const float4*>(&red[w][t * 64 + 4 * j4]));
      *reinterpret_cast<float4*>(P + (ch * T + t0 + t) * RP + 64 * jb + 4 * j4) = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// rowdot reduction: v[t][j] = sum over chunks (in chunk order), then any of
//   f32      [T][r]  fp32 result
//   row_hi/lo[T][RP] bf16 split of scale_row * v (zero for j >= r)
//   t_hi/lo  [RP][TP] bf16 split of v, transposed (zero outside T x r)
//   side -> side_hi/lo: the same transposed split of an extra fp32 [T][r]
//   matrix (XA in the backward pass), since it covers the same tile.
// Workgroup = a 16 t x 64 j tile; thread q handles 4 consecutive j of one t.
// The grid covers T rounded up to 64, so the planes are written (with
// zeros past T) over their whole width TP.
// ---------------------------------------------------------------------------
constexpr int kRedRows = 16;
__global__ __launch_bounds__(256) void rowdot_reduce_kernel(RowdotOuts outs, RowdotJobs jobs, int64_t T, int r,
                                                            int RP, int nc) {
  constexpr int kPad = kRedRows + 8;
  __shared__ __align__(16) uint16_t tr[4][64 * kPad];  // [plane][j][t]
  // grid.y = jobs x j-blocks; the job of this workgroup is uniform
  const int nj = RP / 64;
  const int job = __builtin_amdgcn_readfirstlane((int)blockIdx.y / nj);
  const RowdotOut& o = outs.o[job];
  const float* __restrict__ P = jobs.P[job];
  const int64_t t0 = (int64_t)blockIdx.x * kRedRows;
  const int jb = (int)blockIdx.y - job * nj;
  const bool want_t = o.t_hi != nullptr, want_side = o.side != nullptr;
  if (blockIdx.x == 0 && jb == 0)
    for (int64_t i = threadIdx.x; i < o.nzero; i += 256) o.zero[i] = 0;
  {
    const int q = threadIdx.x;
    const int t = q >> 4, j = 64 * jb + 4 * (q & 15);
    const int64_t tg = t0 + t;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tg < T) {
      // The chunks' loads of a batch are issued together (chunks past nc
      // read zero through an out-of-range offset, no branch), then added in
      // chunk order.
      const rsrc_t rp = make_rsrc(P, (int64_t)nc * T * RP * 4);
      float4 part[8];
      for (int c0 = 0; c0 < nc; c0 += 8) {
        const int n = nc - c0 < 8 ? nc - c0 : 8;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          part[c] = buf_load_f4(rp, off_if(c < n, (uint32_t)((((int64_t)(c0 + c) * T + tg) * RP + j) * 4)));
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c < n) v = (c0 + c == 0) ? part[c] : add4(v, part[c]);
      }
      if (o.f32 && j < r) *reinterpret_cast<float4*>(o.f32 + tg * r + j) = v;
      if (o.row_hi) {
        const float sv[4] = {v.x * o.scale_row, v.y * o.scale_row, v.z * o.scale_row, v.w * o.scale_row};
        const uint32_t h0 = pack_bf16x2(sv[0], sv[1]), h1 = pack_bf16x2(sv[2], sv[3]);
        const uint32_t l0 = pack_bf16x2(sv[0] - bf16_lo(h0), sv[1] - bf16_hi(h0));
        const uint32_t l1 = pack_bf16x2(sv[2] - bf16_lo(h1), sv[3] - bf16_hi(h1));
        *reinterpret_cast<uint2*>(o.row_hi + tg * RP + j) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(o.row_lo + tg * RP + j) = make_uint2(l0, l1);
      }
    }
    if (want_t) {
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h = pack_bf16x2(vv[e], 0.f) & 0xFFFFu;
        const uint32_t l = pack_bf16x2(vv[e] - __uint_as_float(h << 16), 0.f) & 0xFFFFu;
        tr[0][(j - 64 * jb + e) * kPad + t] = (uint16_t)h;
        tr[1][(j - 64 * jb + e) * kPad + t] = (uint16_t)l;
      }
    }
    if (want_side) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tg < T && j < r) x = *reinterpret_cast<const float4*>(o.side + tg * r + j);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h = pack_bf16x2(xv[e], 0.f) & 0xFFFFu;
        const uint32_t l = pack_bf16x2(xv[e] - __uint_as_float(h << 16), 0.f) & 0xFFFFu;
        tr[2][(j - 64 * jb + e) * kPad + t] = (uint16_t)h;
        tr[3][(j - 64 * jb + e) * kPad + t] = (uint16_t)l;
      }
    }
  }
  if (!want_t && !want_side) return;  // uniform per workgroup
  __syncthreads();
  // Tokdot planes: thread q < 128 writes 8 consecutive t of row j, one
  // 16-byte unit of the blocked order.
  if (threadIdx.x < 64 * kRedRows / 8) {
    const int q = threadIdx.x;
    const int j = q / (kRedRows / 8), t8 = 8 * (q % (kRedRows / 8));
    const int64_t jj = 64 * jb + j, tt = t0 + t8;
    const int64_t off = (((tt >> 5) * (RP / 16) + (jj >> 4)) * 64 + (jj & 15) + 16 * ((tt & 31) >> 3)) * 8;
    if (want_t) {
      *reinterpret_cast<u32x4*>(o.t_hi + off) = *reinterpret_cast<const u32x4*>(&tr[0][j * kPad + t8]);
      *reinterpret_cast<u32x4*>(o.t_lo + off) = *reinterpret_cast<const u32x4*>(&tr[1][j * kPad + t8]);
    }
    if (want_side) {
      *reinterpret_cast<u32x4*>(o.side_hi + off) = *reinterpret_cast<const u32x4*>(&tr[2][j * kPad + t8]);
      *reinterpret_cast<u32x4*>(o.side_lo + off) = *reinterpret_cast<const u32x4*>(&tr[3][j * kPad + t8]);
    }
  }
}

// ---------------------------------------------------------------------------
// tokdot partials.  Workgroup = 4 waves = 64 columns m x one chunk of t;
// wave w takes the w-th quarter of the chunk, 32 t per step.  MFMA
// orientation D[j][m]: A operand = S^T from the hi / lo tokdot planes
// (row j = 16 jt + p, 8 consecutive t), B operand = M transposed in
// registers (8 consecutive t of column m = m0 + 4p + c).
// P[c][j][m] has RP rows per chunk.
// ---------------------------------------------------------------------------
template <int JT>
__global__ __launch_bounds__(256) void tokdot_partial_kernel(TokJobs jobs, int64_t TP, int64_t T) {
  __shared__ __align__(16) float red[4][64 * 64];
  constexpr int RP = 16 * JT;
  // Workgroups [wg_begin[j], wg_begin[j + 1]) serve job j (uniform).
  int jsel = 0;
#pragma unroll
  for (int j = 1; j < kTokJobsMax; ++j)
    if (j < jobs.count && (int)blockIdx.x >= jobs.wg_begin[j]) jsel = j;
  const int bid = (int)blockIdx.x - jobs.wg_begin[jsel];
  const TokJob& jb = jobs.j[jsel];
  const uint16_t* __restrict__ M = jb.M;
  const uint16_t* __restrict__ Sh = jb.Sh;
  const uint16_t* __restrict__ Sl = jb.Sl;
  float* __restrict__ P = jb.P;
  const int64_t C = jb.C, TC = jb.TC;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, p = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)(bid % jb.mtiles) * 64;
  const int64_t ch = bid / jb.mtiles;
  const int64_t tbeg = ch * TC;
  const int64_t tend = tbeg + TC < T ? tbeg + TC : T;
  const int64_t TW = TC / 4;
  const int64_t wt0 = tbeg + wave * TW;
  const int64_t wt1 = wt0 + TW < tend ? wt0 + TW : tend;
  const int nsteps = wt1 > wt0 ? (int)((wt1 - wt0 + 31) / 32) : 0;
  const int64_t m = m0 + 4 * p;
  const bool mv = m < C;  // C % 8 == 0: a 4-group is whole or absent

  f32x4 acc[JT][4];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[jt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Regs {
    uint2 a[8];
    u32x4 h[JT], l[JT];
  };
  // M viewed from this chunk's first token: masked lanes (m past C, t past
  // this wave's range) load zero through an offset past the view.
  const rsrc_t rm = make_rsrc(M + tbeg * C, (tend - tbeg) * C * 2);
  const int wlen = (int)(wt1 - tbeg);  // tokens of this wave's range, counted from the view's first
  auto load = [&](int s, Regs& R) {
    const int64_t t = wt0 + 32 * s + 8 * g;
    const int tl = (int)(t - tbeg);
    const uint32_t base = (uint32_t)((tl * C + m) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      R.a[i] = buf_load8(rm, off_if(mv && tl + i < wlen, base + (uint32_t)(i * C * 2)));
    // The planes are zero for t >= T and hold TP >= T tokens, so the loads
    // need no token mask; steps past this wave's range (masked via M) read
    // the chunk's first block.  Each load is 1 KB of consecutive bytes.
    const int64_t blk = (t < tend ? t : tbeg) >> 5;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int64_t off = ((blk * JT + jt) * 64 + lane) * 8;
      R.h[jt] = *reinterpret_cast<const u32x4*>(Sh + off);
      R.l[jt] = *reinterpret_cast<const u32x4*>(Sl + off);
    }
  };
  auto compute = [&](const Regs& R) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 mop = column_of(R.a, c);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        acc[jt][c] = mfma16(as_bf16x8(R.h[jt]), mop, acc[jt][c]);
        acc[jt][c] = mfma16(as_bf16x8(R.l[jt]), mop, acc[jt][c]);
      }
    }
  };

  // Ring of D register sets, as in the rowdot partials.
  constexpr int D = 2;
  Regs R[D];
#pragma unroll
  for (int k = 0; k < D - 1; ++k) load(k, R[k]);
  for (int s = 0; s < nsteps; s += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load(s + k + D - 1, R[(k + D - 1) % D]);
      compute(R[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // D[j][m]: lane holds rows j = 16 jt + 4g + i, column m = m0 + 4p + c.
  // A job whose tokens form one chunk writes its output here (bf16 of
  // scale x sum, the value the reduction would give); otherwise the
  // chunk's fp32 tile goes to P.
  const bool direct = jb.nc == 1;
  const bool m_major = jb.m_major != 0;
  uint16_t* __restrict__ out = jb.out;
  const float sc = jb.scale;
  const int r = jobs.r;
#pragma unroll
  for (int ib = 0; ib < RP / 64 + (RP % 64 ? 1 : 0); ++ib) {
    if (ib) __syncthreads();
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (4 * ib + jt >= JT) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * jt + 4 * g + i;
        const f32x4* a = acc[4 * ib + jt];
        *reinterpret_cast<float4*>(&red[wave][j * 64 + 4 * p]) = make_float4(a[0][i], a[1][i], a[2][i], a[3][i]);
      }
    }
    __syncthreads();
    const int rows = RP - 64 * ib < 64 ? RP - 64 * ib : 64;
    uint2 packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = threadIdx.x + 256 * k;
      const int j = q >> 4, m4 = q & 15;
      float4 sum = *reinterpret_cast<const float4*>(&red[0][j * 64 + 4 * m4]);
#pragma unroll
      for (int w = 1; w < 4; ++w) sum = add4(sum, *reinterpret_cast<const float4*>(&red[w][j * 64 + 4 * m4]));
      packed[k] = make_uint2(pack_bf16x2(sum.x * sc, sum.y * sc), pack_bf16x2(sum.z * sc, sum.w * sc));
      if (j >= rows || m0 + 4 * m4 >= C) continue;
      if (!direct) {
        *reinterpret_cast<float4*>(P + (ch * RP + 64 * ib + j) * C + m0 + 4 * m4) = sum;
      } else if (!m_major && 64 * ib + j < r) {
        *reinterpret_cast<uint2*>(out + (64 * ib + j) * C + m0 + 4 * m4) = packed[k];
      }
    }
    if (direct && m_major) {  // uniform per workgroup
      // Transpose the 64 j x 64 m bf16 tile through LDS so that each
      // thread stores 8 consecutive j of one row m of out [C][r].
      uint16_t* tr = reinterpret_cast<uint16_t*>(&red[0][0]);  // [m][j], j padded to 72
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = threadIdx.x + 256 * k;
        const int j = q >> 4, m4 = q & 15;
        tr[(4 * m4 + 0) * 72 + j] = (uint16_t)(packed[k].x & 0xFFFFu);
        tr[(4 * m4 + 1) * 72 + j] = (uint16_t)(packed[k].x >> 16);
        tr[(4 * m4 + 2) * 72 + j] = (uint16_t)(packed[k].y & 0xFFFFu);
        tr[(4 * m4 + 3) * 72 + j] = (uint16_t)(packed[k].y >> 16);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = threadIdx.x + 256 * k;
        const int mm = q >> 3, j8 = 8 * (q & 7);
        if (m0 + mm < C && j8 < rows && 64 * ib + j8 < r)
          *reinterpret_cast<u32x4*>(out + (m0 + mm) * r + 64 * ib + j8) =
              *reinterpret_cast<const u32x4*>(&tr[mm * 72 + j8]);
      }
    }
  }
}

// out = bf16(s * sum over chunks of P[c][j][m]), stored [j][m] (dB: [r,N]) or
// [m][j] (dA: [K,r]).  Workgroup = a 64 j x 16 m tile; thread q handles 4
// consecutive m of one j.
__global__ __launch_bounds__(256) void tokdot_reduce_kernel(TokJobs jobs, int r, int RP) {
  // Workgroups [red_begin[j], red_begin[j + 1]) serve job j (uniform).
  int jsel = 0;
#pragma unroll
  for (int j = 1; j < kTokJobsMax; ++j)
    if (j < jobs.count && (int)blockIdx.x >= jobs.red_begin[j]) jsel = j;
  const int bid = (int)blockIdx.x - jobs.red_begin[jsel];
  const TokJob& job = jobs.j[jsel];
  const float* __restrict__ P = job.P;
  uint16_t* __restrict__ out = job.out;
  const int64_t C = job.C;
  const int nc = job.nc;
  const float s = job.scale;
  const int m_major = job.m_major;
  const int mt16 = (int)((C + 15) / 16);
  __shared__ __align__(16) uint16_t tr[16 * 72];  // [m][j], j padded to 72
  const int64_t m0 = (int64_t)(bid % mt16) * 16;
  const int jb = bid / mt16;
  const int q = threadIdx.x;
  const int j = q >> 2, m4 = 4 * (q & 3);
  const int jg = 64 * jb + j;
  const int64_t mg = m0 + m4;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (jg < r && mg < C) {
    // Loads of a batch issued together (past nc: zero, no branch), then
    // added in chunk order.
    const rsrc_t rp = make_rsrc(P, (int64_t)nc * RP * C * 4);
    float4 part[8];
    for (int c0 = 0; c0 < nc; c0 += 8) {
      const int n = nc - c0 < 8 ? nc - c0 : 8;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        part[c] = buf_load_f4(rp, off_if(c < n, (uint32_t)((((int64_t)(c0 + c) * RP + jg) * C + mg) * 4)));
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < n) v = (c0 + c == 0) ? part[c] : add4(v, part[c]);
    }
  }
  const uint32_t p0 = pack_bf16x2(v.x * s, v.y * s), p1 = pack_bf16x2(v.z * s, v.w * s);
  if (!m_major) {
    if (jg < r && mg < C) *reinterpret_cast<uint2*>(out + (int64_t)jg * C + mg) = make_uint2(p0, p1);
    return;  // uniform per launch
  }
  tr[(m4 + 0) * 72 + j] = (uint16_t)(p0 & 0xFFFFu);
  tr[(m4 + 1) * 72 + j] = (uint16_t)(p0 >> 16);
  tr[(m4 + 2) * 72 + j] = (uint16_t)(p1 & 0xFFFFu);
  tr[(m4 + 3) * 72 + j] = (uint16_t)(p1 >> 16);
  __syncthreads();
  // Thread q writes 4 consecutive j of row m.
  const int mm = q >> 4, j4 = 4 * (q & 15);
  if (m0 + mm < C && 64 * jb + j4 < r)
    *reinterpret_cast<uint2*>(out + (m0 + mm) * r + 64 * jb + j4) = *reinterpret_cast<const uint2*>(&tr[mm * 72 + j4]);
}

// Zero-fill (used for dA / dB when there are no tokens).
__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_rowdot_batch(int count, const uint16_t* const* M, const uint16_t* const* V, bool v_lr,
                               float* const* P, const RowdotOut* o, int64_t T, int64_t L, int r, int64_t LC,
                               hipStream_t s) {
  if (count < 1 || count > kRowdotJobsMax) return hipErrorInvalidValue;
  const int64_t nc = cdiv(L, LC);
  const int JB = r > 64 ? 2 : 1;
  RowdotJobs jobs{};
  RowdotOuts outs{};
  jobs.nc = (int)nc;
  for (int i = 0; i < count; ++i) {
    jobs.M[i] = M[i];
    jobs.V[i] = V[i];
    jobs.P[i] = P[i];
    outs.o[i] = o[i];
  }
  dim3 grid((unsigned)cdiv(T, 64), (unsigned)(nc * count));
  {
    KernelTimer kt_("rowdot_partial_kernel", s);
    if (v_lr) {
      if (JB == 1) hipLaunchKernelGGL((rowdot_partial_kernel<true, 1>), grid, dim3(256), 0, s, jobs, T, L, r, LC);
      else hipLaunchKernelGGL((rowdot_partial_kernel<true, 2>), grid, dim3(256), 0, s, jobs, T, L, r, LC);
    } else {
      if (JB == 1) hipLaunchKernelGGL((rowdot_partial_kernel<false, 1>), grid, dim3(256), 0, s, jobs, T, L, r, LC);
      else hipLaunchKernelGGL((rowdot_partial_kernel<false, 2>), grid, dim3(256), 0, s, jobs, T, L, r, LC);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("rowdot_reduce_kernel", s);
    hipLaunchKernelGGL(rowdot_reduce_kernel, dim3((unsigned)(cdiv(T, 64) * (64 / kRedRows)), (unsigned)(JB * count)),
                       dim3(256), 0, s, outs, jobs, T, r, 64 * JB, (int)nc);
  }
  return hipGetLastError();
}

hipError_t launch_rowdot(const uint16_t* M, const uint16_t* V, bool v_lr, float* P, const RowdotOut& o, int64_t T,
                         int64_t L, int r, int64_t LC, hipStream_t s) {
  return launch_rowdot_batch(1, &M, &V, v_lr, &P, &o, T, L, r, LC, s);
}

hipError_t launch_tokdot_n(int count, const TokJob* in, int64_t T, int64_t TP, int r, hipStream_t s) {
  if (count < 1 || count > kTokJobsMax) return hipErrorInvalidValue;
  TokJobs jobs{};
  jobs.count = count;
  int nwg = 0, nred = 0;
  const int jbs = (int)cdiv(r, 64);
  for (int i = 0; i < count; ++i) {
    TokJob j = in[i];
    j.nc = (int)cdiv(T, j.TC);
    j.mtiles = (int)cdiv(j.C, 64);
    jobs.j[i] = j;
    jobs.wg_begin[i] = nwg;
    jobs.red_begin[i] = nred;
    nwg += j.mtiles * j.nc;
    if (j.nc > 1) nred += (int)cdiv(j.C, 16) * jbs;  // one chunk: written by the partial kernel
  }
  jobs.r = r;
  const int JT = cdiv(r, 16) <= 4 ? 4 : 8;
  {
    KernelTimer kt_("tokdot_partial_kernel", s);
    if (JT == 4) hipLaunchKernelGGL(tokdot_partial_kernel<4>, dim3((unsigned)nwg), dim3(256), 0, s, jobs, TP, T);
    else hipLaunchKernelGGL(tokdot_partial_kernel<8>, dim3((unsigned)nwg), dim3(256), 0, s, jobs, TP, T);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nred == 0) return hipSuccess;
  {
    KernelTimer kt_("tokdot_reduce_kernel", s);
    hipLaunchKernelGGL(tokdot_reduce_kernel, dim3((unsigned)nred), dim3(256), 0, s, jobs, r, 16 * JT);
  }
  return hipGetLastError();
}

hipError_t launch_tokdot2(const TokJob& a, const TokJob& b, int64_t T, int64_t TP, int r, hipStream_t s) {
  const TokJob j[2] = {a, b};
  return launch_tokdot_n(2, j, T, TP, r, s);
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
