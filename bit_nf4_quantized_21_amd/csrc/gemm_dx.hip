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
//    columns (4 k for all 8 rows at a time).  The codebook is read from a
//    256-entry pair table at LDS address 0 (one 8-byte read per code byte,
//    addressed by one byte-select shift).  The 8 per-row scales of a patch come from a table
//    that the workgroup fills one step earlier, one fp64-exact scale per
//    thread.
//  * dY tiles are staged in LDS in their natural [t][n] layout from
//    registers; codes and dY are loaded two steps ahead.
//  * LDS rows are 128 bytes; the 16-byte chunk index is XOR-ed with bits of
//    (row >> 1) ^ (row >> 4): MFMA operand reads (16 consecutive rows) are
//    conflict-free and the transposed writes (rows 8 apart, all of one
//    parity) are 2-way, the least their parity allows.
//  * Software pipeline: while the MFMAs of step j run on buffers j % 2, the
//    patch of step j+1 is decoded (its first lookups already in the last
//    slices of step j-1) and written with dY(j+1) into buffers (j+1) % 2;
//    one barrier per step, three quarters into it, after which the next
//    step's first operands are read.  A step is 64 slices, each one MFMA
//    plus a fixed share of the operand reads, lookups, packs, LDS writes and
//    global loads, fenced from the next slice so the issue order stays
//    interleaved; q8 / s2 are fetched a step before their scale is stored.
//  * The adapter term is two more steps: A (rows k) against the bf16 hi and
//    lo planes of s G (rows t), staged into the same buffers.
//  * Workgroup order is XCD-aware: each XCD takes a contiguous run of
//    token-tile-major tiles, so the dY rows of a token tile are fetched into
//    that XCD's L2 once and re-read there by every k-tile (measured faster
//    than k-tile-major, which shares the code columns instead).
#include "common.hpp"
#include "timing.hpp"
#include "gemm.hpp"
#include "splitk.hpp"

#include <type_traits>
#include <utility>

namespace qlora {

namespace {
constexpr int kTileK = 256;
constexpr int kTileT = 256;
constexpr int kBuf = 256 * 128;  // 256 rows x 64 bf16
constexpr int kLut = 3072;       // codebook pair table at address 0, 16-entry codebook at 2048
constexpr int kW0 = kLut, kW1 = kW0 + kBuf, kD0 = kW1 + kBuf, kD1 = kD0 + kBuf, kS0 = kD1 + kBuf;
constexpr int kSBytes = 4 * 64 * 4;  // [4 k-blocks][64 rows] fp32 scales
constexpr int kSmem = kS0 + 2 * kSBytes;
constexpr int kCodeStage = 64 * 128;  // raw codes of a step: 64 rows x 256 k
static_assert(kS0 >= 256 * 512, "the dX staging tile fits below the scale tables");

// Calls f(integral_constant<int, I0 + i>) for i = 0, 1, ...: one straight-line
// copy of the slice body per slice, with the slice index a constant.
template <int I0, class F, int... Is>
__device__ __forceinline__ void run_slices(F& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, I0 + Is>{}), ...);
}

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (((row >> 1) ^ (row >> 4)) & 7)) << 4));
}

}  // namespace

__global__ __launch_bounds__(256, 1) void gemm_dx_kernel(DxGemmParams p, Codebook cb) {
  __shared__ __align__(1024) unsigned char smem[kSmem];
  // Raw code tiles of two steps, each its own object so the compiler can
  // tell the stage being filled by buffer-to-LDS loads from the one read.
  __shared__ __align__(1024) unsigned char cst0[kCodeStage], cst1[kCodeStage];
  const int tid = threadIdx.x;

  // Workgroups are dispatched round-robin over the 8 XCDs; each XCD works
  // through its own contiguous run of tiles (whole tiles first, then the
  // contraction slices of the rest), so the slices of a tile share an L2.
  const TileItem it = decode_item(p.plan, blockIdx.x);
  if (it.tile < 0) return;  // uniform per workgroup, before any barrier
  // Tiles are numbered problem-major over the batch.
  const int tile_g = __builtin_amdgcn_readfirstlane(it.tile), sidx = __builtin_amdgcn_readfirstlane(it.sidx);
  const int bat = __builtin_amdgcn_readfirstlane(tile_g / p.tiles_per);
  const int tile = tile_g - bat * p.tiles_per;
  const DxGemmProblem& P = p.prob[bat];
  // Workgroup-uniform values kept in scalar registers (the buffer views
  // built from them must be uniform).
  const int tk = __builtin_amdgcn_readfirstlane(tile % p.tiles_k);
  const int tt = __builtin_amdgcn_readfirstlane(tile / p.tiles_k);
  const float* const lut16 = reinterpret_cast<const float*>(smem + 2048);
  codebook_to_lds(reinterpret_cast<float*>(smem + 2048), cb, tid);

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
  const rsrc_t rc = make_rsrc(P.codes, N * K2);
  const rsrc_t rq = make_rsrc(P.q8, N * bpr);
  const rsrc_t rs = make_rsrc(P.s2, ((N * bpr + 255) / 256) * 4);
  const rsrc_t rd = make_rsrc(P.dY + t0 * N, (T - t0) * N * 2);
  const uint32_t coff = (uint32_t)((8 * rg) * K2 + kcol / 2);
  auto load_code = [&](int j, int i) -> uint32_t { return buf_load4(rc, coff + (uint32_t)(j * 64 * K2 + i * K2)); };
  // Codes of later steps go through LDS: wave w copies rows 16w .. 16w+15
  // of a step (two buffer-to-LDS loads of 8 rows x 128 bytes, load q taking
  // rows 16w + 8q ..) and later reads only those rows, so no barrier orders
  // the copy.  Physical row pr holds row pr ^ ((pr >> 3) & 1): the two rows
  // a wave reads at once (8 apart) sit in opposite halves of the banks.
  const int crow = lane >> 3, cchunk = lane & 7;
  auto dma_codes = [&](unsigned char* st, int j, int q) {
    const int lr = (16 * wave + 8 * q + crow) ^ q;
    buf_load16_to_lds(rc, st + (16 * wave + 8 * q) * 128,
                      (uint32_t)(((int64_t)j * 64 + lr) * K2 + k0 / 2 + 16 * cchunk));
  };
  auto read_code = [&](const unsigned char* st, int i) -> uint32_t {
    const int lr = 8 * rg + i, pr = lr ^ ((lr >> 3) & 1);
    return *reinterpret_cast<const uint32_t*>(st + pr * 128 + 4 * kq);
  };
  // q8 of this thread's scale entry (zero for a k-block past K: its offset
  // is pushed out of the view, so no select has to wait for the load) and
  // its s2.
  auto load_q = [&](int j) -> uint32_t {
    return buf_load1(rq, off_if(sval, (uint32_t)(((int64_t)j * 64 + sr) * bpr + skb)));
  };
  auto load_s = [&](int j) -> float {
    const int64_t b = ((int64_t)j * 64 + sr) * bpr + skb;
    return __uint_as_float(buf_load4(rs, (uint32_t)((b >> 8) * 4)));
  };
  // Columns n >= N of the last step read the next row (or zero past the
  // end): finite values that meet zero W' rows.
  const uint32_t doff = (uint32_t)(xr * N * 2 + 16 * xc);
  auto load_dy = [&](int j, int i) -> u32x4 { return buf_load16(rd, doff + (uint32_t)(j * 128 + i * 32 * N * 2)); };
  auto store_row = [&](int base, int i, const u32x4& v) {
    *reinterpret_cast<u32x4*>(smem + base + swz(xr + 32 * i, xc)) = v;
  };
  auto scale_slot = [&](int sbuf) { return reinterpret_cast<float*>(smem + kS0 + sbuf * kSBytes) + sb * 64 + sr; };
  auto read_scales = [&](int sbuf, int half, float(&sc)[8]) {
    const float* t = reinterpret_cast<const float*>(smem + kS0 + sbuf * kSBytes) + (kq >> 3) * 64 + 8 * rg;
    const float4 v = *reinterpret_cast<const float4*>(t + 4 * half);
    sc[4 * half] = v.x; sc[4 * half + 1] = v.y; sc[4 * half + 2] = v.z; sc[4 * half + 3] = v.w;
  };
  // Column c of patch half hf (k = 8 kq + 4 hf + c, rows 8 rg .. 8 rg + 7)
  // as one 16-byte LDS write.
  auto write_col = [&](int base, int hf, int c, const uint32_t(&col)[4]) {
    *reinterpret_cast<u32x4*>(smem + base + swz(8 * kq + 4 * hf + c, rg)) = u32x4{col[0], col[1], col[2], col[3]};
  };
  // MFMA operand r of a substep s: r < 4 the dY rows 128 wt + 32 r (B), else
  // the W' rows 128 wk + 32 (r - 4) (A); lane half h takes n 8 (2s + h) ..
  auto read_op = [&](int wbase, int dbase, int s, int r) -> bf16x8 {
    return r < 4 ? *reinterpret_cast<const bf16x8*>(smem + dbase + swz(128 * wt + 32 * r + l32, 2 * s + h))
                 : *reinterpret_cast<const bf16x8*>(smem + wbase + swz(128 * wk + 32 * (r - 4) + l32, 2 * s + h));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  uint32_t cA[8], cB[8];    // codes of two steps, alternating
  u32x4 dyr[8];             // dY rows of the next step
  uint32_t qv[2];           // q8 / s2 loaded one step before their scale is stored
  float s2v[2];
  float sc[8];              // scales of the patch being decoded
  float fp[8][8];           // codebook values per decode unit
  uint32_t col[2][4][4];    // packed columns of the two patch halves
  bf16x8 oa[2][4], ob[2][4];

  // The decode of W'(j+1) (codes CN) is cut into 8 units of 2 rows x 4 k:
  // unit u = (half u >> 2, row pair u & 3).  Its 32 lookups g of the pair
  // table (two codebook values each) run at slots 3g/2, its packs 4 slots
  // after the unit's last lookup; slot U of W'(j+1) is slice U - 12 of step
  // j (the first 12 slots fall in the last slices of step j-1).  A slice is
  // one MFMA plus its share of: operand reads for the next substep (slices
  // 0..7 of each substep; the next step's after the barrier at slice 50),
  // lookups, packs, column writes (half 0 at 19..22, half 1 at 43..46), dY
  // rows to LDS (24..31) and from memory (32..39), codes of step j+2
  // (0..7), q8/s2 of step j+3 (8, 9), the scale of W'(j+2) (28, stored at
  // 30) and the scale reads of W'(j+2) (56, 57).  Each slice is fenced so
  // the issue order stays interleaved.
#define QLORA_DX_DECODE_SLOT(U, CODES)                                                                  \
  {                                                                                                    \
    constexpr int U_ = (U);                                                                            \
    constexpr int g_ = (2 * U_ + 2) / 3;                                                               \
    if constexpr (U_ >= 0 && g_ < 32 && (3 * g_) / 2 == U_) {                                          \
      constexpr int u_ = g_ >> 2, w_ = g_ & 3, hf_ = u_ >> 2, pr_ = u_ & 3;                            \
      constexpr int rs_ = w_ >> 1, b_ = w_ & 1;                                                        \
      const float2 v_ = *reinterpret_cast<const float2*>(smem + byte_x8(CODES[2 * pr_ + rs_], 2 * hf_ + b_)); \
      fp[u_][4 * rs_ + 2 * b_] = v_.x;                                                                 \
      fp[u_][4 * rs_ + 2 * b_ + 1] = v_.y;                                                             \
    }                                                                                                  \
    _Pragma("unroll") for (int u_ = 0; u_ < 8; ++u_) {                                                 \
      const int c_ = U_ - (6 * u_ + 8);                                                                \
      if (c_ >= 0 && c_ < 4) {                                                                         \
        const int pr_ = u_ & 3;                                                                        \
        col[u_ >> 2][c_ & 3][pr_] = pack_bf16x2(fp[u_][c_ & 3] * sc[2 * pr_], fp[u_][4 + (c_ & 3)] * sc[2 * pr_ + 1]); \
      }                                                                                                \
    }                                                                                                  \
  }
#define QLORA_DX_SLICE(I, MF, J, WB, DB, WN, DN, SN, SF, CN, CF, QL, QS, CR, CD)                                    \
  {                                                                                                    \
    constexpr int I_ = (I), s_ = I_ >> 4, i_ = I_ & 15;                                                \
    if constexpr (I_ == 50) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                      \
    if constexpr (MF) acc[i_ >> 2][i_ & 3] = mfma32(oa[s_ & 1][i_ >> 2], ob[s_ & 1][i_ & 3], acc[i_ >> 2][i_ & 3]); \
    if constexpr (s_ < 3 && i_ < 8) {                                                                            \
      const bf16x8 v_ = read_op(WB, DB, s_ + 1, i_);                                                   \
      if constexpr (i_ < 4) ob[(s_ + 1) & 1][i_] = v_; else oa[(s_ + 1) & 1][i_ - 4] = v_;                        \
    }                                                                                                  \
    if constexpr (I_ >= 50 && I_ < 58) {                                                                         \
      const bf16x8 v_ = read_op(WN, DN, 0, I_ - 50);                                                   \
      if constexpr (I_ - 50 < 4) ob[0][I_ - 50] = v_; else oa[0][I_ - 54] = v_;                                   \
    }                                                                                                  \
    if constexpr (I_ == 56 || I_ == 57) read_scales(SF, I_ - 56, sc);                                            \
    if constexpr (I_ + 12 >= 12 && I_ + 12 < 54) QLORA_DX_DECODE_SLOT(I_ + 12, CN)                                \
    if constexpr (I_ >= 52) QLORA_DX_DECODE_SLOT(I_ - 52, CF)                                                    \
    if constexpr (I_ >= 19 && I_ < 23) write_col(WN, 0, I_ - 19, col[0][I_ - 19]);                                \
    if constexpr (I_ >= 43 && I_ < 47) write_col(WN, 1, I_ - 43, col[1][I_ - 43]);                                \
    if constexpr (I_ >= 24 && I_ < 32) store_row(DN, I_ - 24, dyr[I_ - 24]);                                     \
    if constexpr (I_ >= 32 && I_ < 40) dyr[I_ - 32] = load_dy((J) + 2, I_ - 32);                                 \
    if constexpr (I_ < 2) dma_codes(CD, (J) + 3, I_);                                                            \
    if constexpr (I_ == 50 || I_ == 51) {                                                              \
      _Pragma("unroll") for (int ii_ = 0; ii_ < 4; ++ii_) CF[4 * (I_ - 50) + ii_] = read_code(CR, 4 * (I_ - 50) + ii_); \
    }                                                                                                  \
    if constexpr (I_ == 8) qv[QL] = load_q((J) + 3);                                                             \
    if constexpr (I_ == 9) s2v[QL] = load_s((J) + 3);                                                            \
    if constexpr (I_ == 28) sfv = dq_scale(qv[QS], s2v[QS]);                                                     \
    if constexpr (I_ == 30) *scale_slot(SF) = sfv;                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
  }
  // Step J on buffers WB/DB (W'(J), dY(J)); WN/DN receive W'(J+1), dY(J+1);
  // scale table SN holds W'(J+1)'s scales, SF receives W'(J+2)'s; CN holds
  // codes(J+1), CF receives codes(J+2); q8/s2 of step J+3 go to set QL, the
  // set QS (loaded one step earlier) gives W'(J+2)'s scale.
#define QLORA_DX_STEP(J, I0, WB, DB, WN, DN, SN, SF, CN, CF, QL, QS, CR, CD)                                    \
  {                                                                                                    \
    float sfv = 0.0f;                                                                                  \
    auto slice_ = [&](auto ic_) __attribute__((always_inline)) {                                       \
      constexpr int I = decltype(ic_)::value;                                                          \
      QLORA_DX_SLICE(I, (I0) == 0, J, WB, DB, WN, DN, SN, SF, CN, CF, QL, QS, CR, CD)                          \
    };                                                                                                 \
    run_slices<(I0)>(slice_, std::make_integer_sequence<int, 64 - (I0)>{});                            \
    (void)sfv;                                                                                         \
  }

  // Prologue.  W'(jbeg) and dY(jbeg) go to buffers 0 directly; the scales of
  // W'(jbeg) and W'(jbeg+1) to tables 0 and 1; dY(jbeg+1) and the q8/s2 of
  // jbeg+2 stay in registers.  Then the last 14 slices of a step jbeg-1
  // read the operands of step jbeg's substep 0, the scales of W'(jbeg+1)
  // and start its decode from codes(jbeg+1) (slices of step jbeg-1 do no
  // loads or LDS writes).
  {
    uint32_t c0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c0[i] = load_code(jbeg, i);
    dma_codes(cst1, jbeg + 1, 0);
    dma_codes(cst1, jbeg + 1, 1);
    dma_codes(cst0, jbeg + 2, 0);
    dma_codes(cst0, jbeg + 2, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) dyr[i] = load_dy(jbeg, i);
    *scale_slot(0) = dq_scale(load_q(jbeg), load_s(jbeg));
    *scale_slot(1) = dq_scale(load_q(jbeg + 1), load_s(jbeg + 1));
    qv[1] = load_q(jbeg + 2);
    s2v[1] = load_s(jbeg + 2);
    __syncthreads();  // codebook, scale tables
    pair_table_to_lds(smem, lut16, tid);  // visible after the prologue's second barrier
    float s0[8];
    read_scales(0, 0, s0);
    read_scales(0, 1, s0);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t cw[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const int nib = 4 * hf + c;  // nibble of the code dword = k offset in the patch
          const float fa = lut16[(c0[2 * pr] >> (4 * nib)) & 15u];
          const float fb = lut16[(c0[2 * pr + 1] >> (4 * nib)) & 15u];
          cw[pr] = pack_bf16x2(fa * s0[2 * pr], fb * s0[2 * pr + 1]);
        }
        write_col(kW0, hf, c, cw);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) store_row(kD0, i, dyr[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dyr[i] = load_dy(jbeg + 1, i);
    __syncthreads();  // W'(jbeg), dY(jbeg) complete
  }
  QLORA_DX_STEP(jbeg - 1, 50, kW1, kD1, kW0, kD0, 0, 1, cA, cB, 0, 1, cst1, cst0)

  // Steps past jend only prefetch and decode data that is never used.
  int j = jbeg;
  for (; j + 2 <= jend; j += 2) {
    QLORA_DX_STEP(j, 0, kW0, kD0, kW1, kD1, 1, 0, cB, cA, 0, 1, cst0, cst1)
    QLORA_DX_STEP(j + 1, 0, kW1, kD1, kW0, kD0, 0, 1, cA, cB, 1, 0, cst1, cst0)
  }
  if (j < jend) QLORA_DX_STEP(j, 0, kW0, kD0, kW1, kD1, 1, 0, cB, cA, 0, 1, cst0, cst1)
#undef QLORA_DX_STEP
#undef QLORA_DX_SLICE
#undef QLORA_DX_DECODE_SLOT
  __syncthreads();  // every wave is done with the buffers

  // Adapter term: A[k][j] (rows k) against the hi and lo rows of s G
  // (rows t), 64 j per pass, carried by slice 0.  The three tiles are copied
  // by buffer-to-LDS loads straight into the swizzled layout: wave w fills
  // rows [64w, 64w+64), 8 rows per instruction, lane l the physical chunk
  // l % 8 of row l / 8 with the logical chunk it holds; chunks past r read
  // zero through an out-of-range offset.
  const int r = p.r;
  if (sidx == 0) {
    const rsrc_t ra = make_rsrc(P.A + k0 * r, (K - k0) * r * 2);
    const rsrc_t rgh = make_rsrc(P.Gh + t0 * p.RP, (T - t0) * p.RP * 2);
    const rsrc_t rgl = make_rsrc(P.Gl + t0 * p.RP, (T - t0) * p.RP * 2);
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
        bf16x8 av[4], bh[4], bl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          av[q] = read_op(kW0, kD0, s, 4 + q);
          bh[q] = read_op(kW0, kD0, s, q);
          bl[q] = read_op(kW0, kD1, s, q);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[a][b] = mfma32(av[a], bh[b], acc[a][b]);
            acc[a][b] = mfma32(av[a], bl[b], acc[a][b]);
          }
      }
    }
  }

  if (it.S > 1 && !splitk_combine(acc, p.slots + (int64_t)it.ordinal * it.S * kSplitSlotFloats,
                                  p.counters + it.ordinal, p.counters + p.plan.nsplit() + it.ordinal, it.S, sidx,
                                  reinterpret_cast<int*>(smem + kS0), p.status))
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
    if (t < T && k < K) *reinterpret_cast<u32x4*>(P.dX + t * K + k) = v;  // K % 64 == 0: chunks whole
  }
}

SplitPlan dx_plan(int64_t T, int64_t K, int64_t N, int batch) {
  return make_split_plan((int64_t)batch * ((K + kTileK - 1) / kTileK) * ((T + kTileT - 1) / kTileT), (N + 63) / 64);
}

hipError_t launch_gemm_dx(const DxGemmParams& p0, const Codebook& cb, hipStream_t s) {
  DxGemmParams p = p0;
  p.batch = 1;
  p.prob[0] = DxGemmProblem{p.dY, p.codes, p.q8, p.s2, p.A, p.Gh, p.Gl, p.dX};
  return launch_gemm_dx_batched(p, cb, s);
}

hipError_t launch_gemm_dx_batched(const DxGemmParams& p0, const Codebook& cb, hipStream_t s) {
  DxGemmParams p = p0;
  p.tiles_k = (int)((p.K + kTileK - 1) / kTileK);
  p.tiles_t = (int)((p.T + kTileT - 1) / kTileT);
  p.tiles_per = p.tiles_k * p.tiles_t;
  p.plan = dx_plan(p.T, p.K, p.N, p.batch);
  {
    KernelTimer kt_("gemm_dx_kernel", s);
    hipLaunchKernelGGL(gemm_dx_kernel, dim3(8 * p.plan.items), dim3(256), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
