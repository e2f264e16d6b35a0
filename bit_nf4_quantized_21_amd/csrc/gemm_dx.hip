// Backward dequantize-GEMM for the input gradient of the frozen NF4 layer,
// with the adapter's rank-r term as one extra contraction step, for gfx950.
//
//   dX^T[k][t] = sum_n W'[n][k] dY[t][n]  +  sum_j A[k][j] (s G[t][j])
//
// i.e. dX = dY W' + s G A^T with G = dY B^T: the gradient flowing through the
// frozen 4-bit weight and through the adapter (QLoRA abstract: backpropagation
// through the frozen 4-bit model into LoRA; the base weight gets no gradient).
// W' = bf16(c[code] * fp32(q8*s2/255)) as in the forward pass.
//
// Design (one workgroup = 4 waves in a 2 x 2 grid = a 256 (k) x 256 (t) tile):
//  * The contraction runs over W's rows n, 64 per step (4 substeps of 16).
//    The MFMA needs 8 consecutive n per lane, but the codes run along k, so
//    W' goes through LDS transposed ([k][n]): each thread decodes an 8 x 8
//    patch (8 rows n, 8 k = one code dword per row) and writes 8 16-byte
//    columns, half of them (4 k for all 8 rows) every two substeps.  The codebook is read from LDS address 0 (one bitfield extract
//    per lookup address).  The 8 per-row scales of a patch come from a table
//    that the workgroup fills one step earlier, one fp64-exact scale per
//    thread.
//  * dY tiles are staged in LDS in their natural [t][n] layout from
//    registers; codes and dY are loaded two steps ahead.
//  * LDS rows are 128 bytes; the 16-byte chunk index is XOR-ed with bits of
//    (row >> 1) ^ (row >> 4): MFMA operand reads (16 consecutive rows) are
//    conflict-free and the transposed writes (rows 8 apart, all of one
//    parity) are 2-way, the least their parity allows.
//  * Software pipeline: while the MFMAs of step j run on buffers j % 2, the
//    patch of step j+1 is decoded (two rows per substep) and written with
//    dY(j+1) into buffers (j+1) % 2; one barrier per step.
//  * The adapter term is two more steps: A (rows k) against the bf16 hi and
//    lo planes of s G (rows t), staged into the same buffers.
//  * Workgroup order is XCD-aware (each XCD takes a contiguous run of
//    k-tile-major tiles, sharing the code columns of one k range).
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"
#include "splitk.hpp"

namespace qlora {

namespace {
constexpr int kTileK = 256;
constexpr int kTileT = 256;
constexpr int kBuf = 256 * 128;  // 256 rows x 64 bf16
constexpr int kLut = 1024;       // codebook slot at address 0
constexpr int kW0 = kLut, kW1 = kW0 + kBuf, kD0 = kW1 + kBuf, kD1 = kD0 + kBuf, kS0 = kD1 + kBuf;
constexpr int kSBytes = 4 * 64 * 4;  // [4 k-blocks][64 rows] fp32 scales
constexpr int kSmem = kS0 + 2 * kSBytes;
static_assert(kS0 >= 256 * 512, "the dX staging tile fits below the scale tables");

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (((row >> 1) ^ (row >> 4)) & 7)) << 4));
}

// Codebook values (table at LDS address 0) of nibbles 4 HF .. 4 HF + 3 of a
// code dword: byte q of (x << 2) & 0x3C3C3C3C is 4 * code(2q), of
// (x >> 2) & 0x3C3C3C3C is 4 * code(2q + 1).
template <int HF>
__device__ __forceinline__ void lut4(const unsigned char* smem, uint32_t x, float (&f)[4]) {
  const uint32_t y4 = (x << 2) & 0x3C3C3C3Cu, z4 = (x >> 2) & 0x3C3C3C3Cu;
  f[0] = *reinterpret_cast<const float*>(smem + bfe<16 * HF, 8>(y4));
  f[1] = *reinterpret_cast<const float*>(smem + bfe<16 * HF, 8>(z4));
  f[2] = *reinterpret_cast<const float*>(smem + bfe<16 * HF + 8, 8>(y4));
  f[3] = *reinterpret_cast<const float*>(smem + bfe<16 * HF + 8, 8>(z4));
}
}  // namespace

__global__ __launch_bounds__(256, 1) void gemm_dx_kernel(DxGemmParams p, Codebook cb) {
  __shared__ __align__(1024) unsigned char smem[kSmem];
  const int tid = threadIdx.x;

  // Workgroups are dispatched round-robin over the 8 XCDs; each XCD works
  // through its own contiguous run of tiles (whole tiles first, then the
  // contraction slices of the rest), so the slices of a tile share an L2.
  const TileItem it = decode_item(p.plan, blockIdx.x);
  if (it.tile < 0) return;  // uniform per workgroup, before any barrier
  const int tile = __builtin_amdgcn_readfirstlane(it.tile), sidx = __builtin_amdgcn_readfirstlane(it.sidx);
  // Workgroup-uniform values kept in scalar registers (the buffer views
  // built from them must be uniform).
  const int tk = __builtin_amdgcn_readfirstlane(tile / p.tiles_t);
  const int tt = __builtin_amdgcn_readfirstlane(tile % p.tiles_t);
  codebook_to_lds(reinterpret_cast<float*>(smem), cb, tid);

  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wk = wave & 1, wt = wave >> 1;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int64_t k0 = (int64_t)tk * kTileK, t0 = (int64_t)tt * kTileT;
  const int64_t K2 = K / 2, bpr = K / 64;
  const int nsteps = (int)((N + 63) / 64);
  const int jbeg = __builtin_amdgcn_readfirstlane(it.kbeg), jend = __builtin_amdgcn_readfirstlane(it.kend);
  (void)nsteps;

  // dY staging: lane -> rows xr + 32 i of the tile, 16-byte chunk xc.
  const int xc = tid & 7, xr = tid >> 3;
  // Patch: rows 8 rg .. 8 rg + 7 of the step, k = k0 + 8 kq .. + 7.
  const int rg = tid >> 5, kq = tid & 31;
  const int64_t kcol = k0 + 8 * kq;
  // Scale table entry of this thread: row sr of the step, k-block sb.
  const int sr = tid & 63, sb = tid >> 6;
  const int64_t skb = k0 / 64 + sb;
  const bool sval = 64 * skb < K;

  // Buffer views: loads past the end return zero.  Codes of rows n >= N
  // read zero and their scales are zero, so those W' rows vanish; k past K
  // has zero scales too.  dY rows are viewed from this tile's first row.
  const rsrc_t rc = make_rsrc(p.codes, N * K2);
  const rsrc_t rd = make_rsrc(p.dY + t0 * N, (T - t0) * N * 2);
  const uint32_t coff = (uint32_t)((8 * rg) * K2 + kcol / 2);
  auto load_codes = [&](int j, uint32_t(&c)[8]) {
    const uint32_t base = coff + (uint32_t)(j * 64 * K2);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = buf_load4(rc, base + (uint32_t)(i * K2));
  };
  auto load_qs = [&](int j, uint32_t& q, float& s2) {
    const int64_t n = (int64_t)j * 64 + sr;
    const bool ok = n < N && sval;
    const int64_t b = n * bpr + skb;
    q = ok ? (uint32_t)p.q8[b] : 0u;
    s2 = ok ? p.s2[b >> 8] : 0.0f;
  };
  auto store_scale = [&](int sbuf, uint32_t q, float s2) {
    reinterpret_cast<float*>(smem + kS0 + sbuf * kSBytes)[sb * 64 + sr] = dq_scale(q, s2);
  };
  // Columns n >= N of the last step read the next row (or zero past the
  // end): finite values that meet zero W' rows.
  const uint32_t doff = (uint32_t)(xr * N * 2 + 16 * xc);
  auto load_dy = [&](int j, u32x4(&v)[8]) {
    const uint32_t base = doff + (uint32_t)(j * 128);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = buf_load16(rd, base + (uint32_t)(i * 32 * N * 2));
  };
  auto store_rows = [&](int base, const u32x4(&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(smem + base + swz(xr + 32 * i, xc)) = v[i];
  };
  auto read_scales = [&](int sbuf, float(&sc)[8]) {
    const float* s = reinterpret_cast<const float*>(smem + kS0 + sbuf * kSBytes) + (kq >> 3) * 64 + 8 * rg;
    const float4 a = *reinterpret_cast<const float4*>(s), b = *reinterpret_cast<const float4*>(s + 4);
    sc[0] = a.x; sc[1] = a.y; sc[2] = a.z; sc[3] = a.w;
    sc[4] = b.x; sc[5] = b.y; sc[6] = b.z; sc[7] = b.w;
  };
  // Half HF of the patch, rows 4 R4 .. 4 R4 + 3: column e = 4 HF + c gets the
  // bf16 pair (row 2q, row 2q+1) as dword q.
#define QLORA_DX_DECODE(HF, R4, CN)                                                    \
  {                                                                                  \
    float f0[4], f1[4], f2[4], f3[4];                                                \
    lut4<HF>(smem, CN[4 * (R4) + 0], f0);                                            \
    lut4<HF>(smem, CN[4 * (R4) + 1], f1);                                            \
    lut4<HF>(smem, CN[4 * (R4) + 2], f2);                                            \
    lut4<HF>(smem, CN[4 * (R4) + 3], f3);                                            \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                  \
      col[c][2 * (R4) + 0] = pack_bf16x2(f0[c] * sc[4 * (R4) + 0], f1[c] * sc[4 * (R4) + 1]); \
      col[c][2 * (R4) + 1] = pack_bf16x2(f2[c] * sc[4 * (R4) + 2], f3[c] * sc[4 * (R4) + 3]); \
    }                                                                                \
  }
  auto write_half = [&](int base, int hf, const uint32_t(&col)[4][4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(smem + base + swz(8 * kq + 4 * hf + c, rg)) =
          u32x4{col[c][0], col[c][1], col[c][2], col[c][3]};
  };
  auto read_ops = [&](int wbase, int dbase, int s, bf16x8(&a)[4], bf16x8(&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const bf16x8*>(smem + wbase + swz(128 * wk + 32 * i + l32, 2 * s + h));
      b[i] = *reinterpret_cast<const bf16x8*>(smem + dbase + swz(128 * wt + 32 * i + l32, 2 * s + h));
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  uint32_t cA[8], cB[8];   // codes, alternating steps
  u32x4 dyr[8];            // dY rows of the next step
  uint32_t qv;
  float s2v;
  float sc[8];
  uint32_t col[4][4];
  bf16x8 oa0[4], ob0[4], oa1[4], ob1[4];

  // Prologue: W'(0), dY(0) in buffers 0; scales of W(1) in table 1; codes(1)
  // and dY(1) in the B registers.
  load_codes(jbeg, cA);
  load_dy(jbeg, dyr);
  load_qs(jbeg, qv, s2v);
  store_scale(0, qv, s2v);
  load_qs(jbeg + 1, qv, s2v);
  store_scale(1, qv, s2v);
  __syncthreads();  // codebook, scale tables
  read_scales(0, sc);
  QLORA_DX_DECODE(0, 0, cA)
  QLORA_DX_DECODE(0, 1, cA)
  write_half(kW0, 0, col);
  QLORA_DX_DECODE(1, 0, cA)
  QLORA_DX_DECODE(1, 1, cA)
  write_half(kW0, 1, col);
  store_rows(kD0, dyr);
  load_codes(jbeg + 1, cB);
  __syncthreads();
  read_ops(kW0, kD0, 0, oa0, ob0);

  // One step on buffers WB/DB (the next step's: WN/DN); the codes of step
  // j+1 are in CN and those of step j+2 are loaded into CF; dY(j+1) is
  // loaded at the top and written in the last substep; the scale table SN
  // holds W(j+1)'s scales and table SF receives W(j+2)'s.
#define QLORA_DX_MFMA(OA, OB)                                                                   \
  _Pragma("unroll") for (int a = 0; a < 4; ++a) {                                               \
    _Pragma("unroll") for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(OA[a], OB[b], acc[a][b]);  \
  }
#define QLORA_DX_SCHED(NW)                                                \
  _Pragma("unroll") for (int i = 0; i < 16; ++i) {                        \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    \
    if (i < (NW)) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);      \
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                    \
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                    \
  }                                                                       \
  __builtin_amdgcn_sched_barrier(0);
#define QLORA_DX_STEP(J, WB, DB, WN, DN, SN, SF, CN, CF)                                                    \
  {                                                                                                        \
    const int j_ = (J);                                                                                    \
    /* qs first: its use later in this step then waits for no newer load */                                \
    load_qs(j_ + 2, qv, s2v);                                                                              \
    load_dy(j_ + 1, dyr);                                                                                  \
    load_codes(j_ + 2, CF);                                                                                \
    read_scales(SN, sc);                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    /* substep 0: columns 0..3 of rows 0..3 of the next patch */                                           \
    read_ops(WB, DB, 1, oa1, ob1);                                                                         \
    QLORA_DX_MFMA(oa0, ob0)                                                                                \
    QLORA_DX_DECODE(0, 0, CN)                                                                              \
    QLORA_DX_SCHED(0)                                                                                      \
    /* substep 1: columns 0..3 of rows 4..7, then those 4 columns to LDS */                                \
    read_ops(WB, DB, 2, oa0, ob0);                                                                         \
    QLORA_DX_MFMA(oa1, ob1)                                                                                \
    QLORA_DX_DECODE(0, 1, CN)                                                                              \
    write_half(WN, 0, col);                                                                                \
    QLORA_DX_SCHED(4)                                                                                      \
    /* substep 2: columns 4..7 of rows 0..3 */                                                             \
    read_ops(WB, DB, 3, oa1, ob1);                                                                         \
    QLORA_DX_MFMA(oa0, ob0)                                                                                \
    QLORA_DX_DECODE(1, 0, CN)                                                                              \
    QLORA_DX_SCHED(0)                                                                                      \
    /* substep 3: columns 4..7 of rows 4..7; dY(j+1), the other patch half */                              \
    /* and W(j+2)'s scale to their buffers */                                                              \
    QLORA_DX_MFMA(oa1, ob1)                                                                                \
    QLORA_DX_DECODE(1, 1, CN)                                                                              \
    write_half(WN, 1, col);                                                                                \
    store_rows(DN, dyr);                                                                                   \
    store_scale(SF, qv, s2v);                                                                              \
    QLORA_DX_SCHED(13)                                                                                     \
    lds_barrier();                                                                                         \
    read_ops(WN, DN, 0, oa0, ob0);                                                                         \
  }

  // Steps past jend only prefetch and decode data that is never used.
  int j = jbeg;
  for (; j + 2 <= jend; j += 2) {
    QLORA_DX_STEP(j, kW0, kD0, kW1, kD1, 1, 0, cB, cA)
    QLORA_DX_STEP(j + 1, kW1, kD1, kW0, kD0, 0, 1, cA, cB)
  }
  if (j < jend) QLORA_DX_STEP(j, kW0, kD0, kW1, kD1, 1, 0, cB, cA)
#undef QLORA_DX_STEP
#undef QLORA_DX_SCHED
#undef QLORA_DX_DECODE
  // Every buffer is free after the last step's barrier.

  // Adapter term: A[k][j] (rows k) against the hi and lo rows of s G
  // (rows t), 64 j per pass, carried by slice 0.  The three tiles are copied
  // by buffer-to-LDS loads straight into the swizzled layout: wave w fills
  // rows [64w, 64w+64), 8 rows per instruction, lane l the physical chunk
  // l % 8 of row l / 8 with the logical chunk it holds; chunks past r read
  // zero through an out-of-range offset.
  const int r = p.r;
  if (sidx == 0) {
    const rsrc_t ra = make_rsrc(p.A + k0 * r, (K - k0) * r * 2);
    const rsrc_t rgh = make_rsrc(p.Gh + t0 * p.RP, (T - t0) * p.RP * 2);
    const rsrc_t rgl = make_rsrc(p.Gl + t0 * p.RP, (T - t0) * p.RP * 2);
    const int drow = lane >> 3, dphys = lane & 7;
    for (int jb = 0; jb < p.RP; jb += 64) {
      __syncthreads();  // every wave is done with the buffers
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + drow;
        const int lchunk = dphys ^ (((row >> 1) ^ (row >> 4)) & 7);
        const int jj = jb + 8 * lchunk;
        const uint32_t ao = jj < r ? (uint32_t)(row * r * 2 + jj * 2) : 0x7FFFFFF0u;
        const uint32_t go = (uint32_t)(row * p.RP * 2 + jj * 2);
        buf_load16_to_lds(ra, smem + kW0 + (64 * wave + 8 * i) * 128, ao);
        buf_load16_to_lds(rgh, smem + kD0 + (64 * wave + 8 * i) * 128, go);
        buf_load16_to_lds(rgl, smem + kD1 + (64 * wave + 8 * i) * 128, go);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        read_ops(kW0, kD0, s, oa0, ob0);
        QLORA_DX_MFMA(oa0, ob0)
        read_ops(kW0, kD1, s, oa1, ob1);
        QLORA_DX_MFMA(oa1, ob1)
      }
    }
  }
#undef QLORA_DX_MFMA

  if (it.S > 1 && !splitk_combine(acc, p.slots + (int64_t)it.ordinal * it.S * kSplitSlotFloats,
                                  p.counters + it.ordinal, it.S, sidx, reinterpret_cast<int*>(smem + kS0)))
    return;

  // dX through LDS: D[k][t] of a 32x32 tile gives lane (l32, h) token
  // t = 128 wt + 32 b + l32 and the 4 features 8 q4 + 4h + (0..3) of k-block
  // 128 wk + 32 a, written as bf16 into a [256 t][256 k] tile whose 16-byte
  // chunks are XOR-swizzled by the row (the 32 lanes of a write land in 32
  // distinct chunks); then each 32 lanes store one whole 512-byte row of dX.
  __syncthreads();  // every wave is done with the operand buffers
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int row = 128 * wt + 32 * b + l32;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 16 * wk + 4 * a + q4;
        const f32x16& v = acc[a][b];
        *reinterpret_cast<uint2*>(smem + row * 512 + ((c ^ l32) << 4) + 8 * h) =
            make_uint2(pack_bf16x2(v[4 * q4 + 0], v[4 * q4 + 1]), pack_bf16x2(v[4 * q4 + 2], v[4 * q4 + 3]));
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int idx = 256 * i + tid, row = idx >> 5, c = idx & 31;
    const int64_t t = t0 + row, k = k0 + 8 * c;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * 512 + ((c ^ (row & 31)) << 4));
    if (t < T && k < K) *reinterpret_cast<u32x4*>(p.dX + t * K + k) = v;  // K % 64 == 0: chunks whole
  }
}

SplitPlan dx_plan(int64_t T, int64_t K, int64_t N) {
  return make_split_plan(((K + kTileK - 1) / kTileK) * ((T + kTileT - 1) / kTileT), (N + 63) / 64);
}

hipError_t launch_gemm_dx(const DxGemmParams& p0, const Codebook& cb, hipStream_t s) {
  DxGemmParams p = p0;
  p.tiles_k = (int)((p.K + kTileK - 1) / kTileK);
  p.tiles_t = (int)((p.T + kTileT - 1) / kTileT);
  p.plan = dx_plan(p.T, p.K, p.N);
  {
    KernelTimer kt_("gemm_dx_kernel", s);
    hipLaunchKernelGGL(gemm_dx_kernel, dim3(8 * p.plan.items), dim3(256), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
