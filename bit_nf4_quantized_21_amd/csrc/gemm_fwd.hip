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
// Design (one workgroup = 4 waves, one per SIMD = a 256 (n) x 256 (m) tile):
//  * K advances one 64-weight quant block per step, so each W row contributes
//    one 32-byte code segment and one scale per step.
//  * W' never touches LDS: lane (row, half h) loads its 16 code bytes and
//    decodes them straight into the MFMA A-operand registers.  Waves
//    partition n, so each W row is decoded once per workgroup and the
//    dequantization cost is amortised over 256 tokens.
//  * Inside a step the contraction runs over a fixed permutation of k: lane
//    half h, substep s, element i covers k = 32h + 8s + i; X is read from
//    LDS in the same permuted order, so the sum is unchanged.
//  * Software pipeline per step (4 substeps x 16 MFMAs): during substep s the
//    X operands of substep s+1 are read from LDS and chunk s of the next
//    step's W is looked up, scaled and packed to bf16, each MFMA carrying a
//    fixed share of that work (a substep is 16 fenced slices).  X tiles go
//    through a 4-stage LDS ring filled by buffer-to-LDS loads issued two
//    steps ahead (no registers, no LDS write instructions); each stage is
//    its own LDS object, so the compiler can tell the stage being filled
//    from the ones being read and puts no wait before the reads.  Codes are
//    loaded two steps ahead into registers.  One barrier per step, before
//    substep 3, waits only for the loads the next step reads (an explicit
//    count leaves the younger ones in flight), so the next step's first
//    operand reads overlap substep 3.
//  * X rows are 128 bytes in LDS with the 16-byte chunk index XOR-ed with
//    bits 1..3 of the row: the 16 rows read by one 16-lane phase land in 16
//    distinct 4-bank groups of gfx950's 64-bank LDS, and the 16 lanes of a
//    write phase cover two adjacent rows, i.e. all 64 banks.
//  * The codebook is held in LDS as a 256-entry pair table at address 0:
//    one 8-byte read per code byte returns the values of two elements, and
//    its address is one byte-select shift of the code dword.
//  * Ragged tiles use buffer loads, which return zero past the end.
//  * Workgroup order is XCD-aware: each XCD works through a contiguous run of
//    token-tile-major tiles, so an X tile is fetched into an XCD's L2 once and
//    re-read from there by every n-tile.
#include "common.hpp"
#include "gemm.hpp"
#include "splitk.hpp"
#include "timing.hpp"

namespace qlora {

namespace {
constexpr int kTileN = 256;
constexpr int kTileM = 256;
constexpr int kStageBytes = kTileM * 128;  // one X stage: 256 rows x 64 bf16
constexpr int kLutBytes = 4096;            // pair table at 0, codebook at 2048, split ticket at 2112
}  // namespace

__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(FwdGemmParams p, Codebook cb) {
  // LDS: the codebook pair table (with the 16-entry codebook and the split
  // ticket after it) and four X stages, each its own object so the compiler
  // can tell a stage being filled by buffer-to-LDS loads from the ones read.
  __shared__ __align__(4096) unsigned char tbl[kLutBytes];
  __shared__ __align__(1024) unsigned char xs0[kStageBytes], xs1[kStageBytes], xs2[kStageBytes], xs3[kStageBytes];
  float* const lut16 = reinterpret_cast<float*>(tbl + 2048);
  unsigned char* const xring[4] = {xs0, xs1, xs2, xs3};
  const int tid = threadIdx.x;

  // Workgroups are dispatched round-robin over the 8 XCDs and each XCD takes
  // a contiguous run of tiles.  With many token tiles the tiles are ordered
  // token-tile-major, so an X tile (re-read by every n-tile) stays in that
  // XCD's L2; with at most two (T <= 512) they are ordered n-tile-major, so
  // the tiles that share an n-tile's codes run together (measured 2.5 %
  // faster at T = 512).
  // Items are (tile, contraction slice) pairs, slices of a tile adjacent.
  const TileItem it = decode_item(p.plan, blockIdx.x);
  if (it.tile < 0) return;  // uniform per workgroup, before any barrier
  // Tiles are numbered problem-major over the batch.
  const int tile_g = __builtin_amdgcn_readfirstlane(it.tile), sidx = __builtin_amdgcn_readfirstlane(it.sidx);
  const int bat = __builtin_amdgcn_readfirstlane(tile_g / p.tiles_per);
  const int tile = tile_g - bat * p.tiles_per;
  const FwdGemmProblem& P = p.prob[bat];
  const bool n_major = p.tiles_m <= 2;
  const int tm = __builtin_amdgcn_readfirstlane(n_major ? tile % p.tiles_m : tile / p.tiles_n);
  const int tn = __builtin_amdgcn_readfirstlane(n_major ? tile / p.tiles_m : tile % p.tiles_n);

  codebook_to_lds(lut16, cb, tid);

  // wave is uniform: readfirstlane lets the compiler keep what derives from it
  // (LDS addresses of the buffer-to-LDS copies, M0) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, ml = lane & 31, h = lane >> 5;
  const int64_t T = p.T, K = p.K, N = p.N;
  const int64_t n0 = (int64_t)tn * kTileN, m0 = (int64_t)tm * kTileM;
  const int64_t K2 = K / 2, bpr = K / 64;
  const int nk = (int)(K / 64);
  const int kbeg = __builtin_amdgcn_readfirstlane(it.kbeg), kend = __builtin_amdgcn_readfirstlane(it.kend);
  auto clampk = [&](int k) { return k < nk ? k : nk - 1; };  // past the end: redundant, in bounds

  // Buffer views of this tile's rows: reads past the last row return zero.
  const rsrc_t rx = make_rsrc(P.X + m0 * K, (T - m0) * K * 2);
  const rsrc_t rc = make_rsrc(P.codes + n0 * K2, (N - n0) * K2);
  const rsrc_t rq = make_rsrc(P.q8 + n0 * bpr, (N - n0) * bpr);
  const rsrc_t rs = make_rsrc(P.s2, ((N * bpr + 255) / 256) * 4);

  int nl[2];
  bool nval[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    nl[g] = 64 * wave + 32 * g + ml;
    nval[g] = n0 + nl[g] < N;
  }

  // X staging by buffer-to-LDS loads: wave w fills rows [64w, 64w+64) of a
  // stage, 8 rows per instruction; lane l writes physical chunk l%8 of row
  // 64w + 8j + l/8 with the logical chunk (l%8) ^ ((row >> 1) & 7) of X.
  const int dr = lane >> 3, dpc = lane & 7;
  const uint32_t xg_even = (uint32_t)((64 * wave + dr) * K * 2 + ((dpc ^ (dr >> 1)) << 4));
  const uint32_t xg_odd = (uint32_t)((64 * wave + dr) * K * 2 + ((dpc ^ ((dr >> 1) | 4)) << 4));
  auto dma_x_row = [&](int stage, int kb, int j) {
    buf_load16_to_lds(rx, xring[stage] + (64 * wave + 8 * j) * 128,
                      ((j & 1) ? xg_odd : xg_even) + (uint32_t)(8 * j * K * 2 + kb * 128));
  };
  // One of the six loads of load_w: part 3g + {0: codes, 1: q8, 2: s2}.
  auto load_w_part = [&](int kb, u32x4(&c)[2], uint32_t(&q)[2], float(&sv)[2], int part) {
    const int g = part / 3;
    if (part % 3 == 0) {
      c[g] = buf_load16(rc, (uint32_t)(nl[g] * K2 + kb * 32 + 16 * h));
    } else if (part % 3 == 1) {
      q[g] = buf_load1(rq, (uint32_t)(nl[g] * bpr + kb));
    } else {
      const int64_t b = (n0 + nl[g]) * bpr + kb;
      sv[g] = __uint_as_float(buf_load4(rs, (uint32_t)((b >> 8) * 4)));
    }
  };
  auto load_w = [&](int kb, u32x4(&c)[2], uint32_t(&q)[2], float(&sv)[2]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      c[g] = buf_load16(rc, (uint32_t)(nl[g] * K2 + kb * 32 + 16 * h));
      q[g] = buf_load1(rq, (uint32_t)(nl[g] * bpr + kb));
      const int64_t b = (n0 + nl[g]) * bpr + kb;
      sv[g] = __uint_as_float(buf_load4(rs, (uint32_t)((b >> 8) * 4)));
    }
  };
  auto lut8 = [&](uint32_t x, float(&f)[8]) { lut8_pairs(tbl, x, f); };
  auto pack8 = [&](const float(&f)[8], float sc) -> bf16x8 {
    return as_bf16x8(pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                     pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc));
  };
  // B operand (X) of substep s: row 32 mi + ml, logical chunk 4h + s.
  const int sw = (ml >> 1) & 7;
  auto read_x = [&](int stage, int s, bf16x8(&xo)[8]) {
    const unsigned char* b = xring[stage] + ml * 128 + (((4 * h + s) ^ sw) << 4);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) xo[mi] = *reinterpret_cast<const bf16x8*>(b + mi * 4096);
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[g][mi][e] = 0.0f;

  u32x4 cA[2], cB[2];           // codes of the next step / the step after
  uint32_t qA[2], qB[2];
  float sA[2], sB[2];
  bf16x8 wc[2][4], wn[2][4];    // W' operands of this step / the next
  float fp[2][8];               // codebook values of a chunk awaiting scale + pack
  bf16x8 xa[8], xb[8];          // X operands, alternating substeps

  // Prologue: the pair table; X(0), X(1) in stages 0, 1; W(0) decoded;
  // then codes(1) and X(2) in flight, issued in the order the loop issues
  // them (codes, then a stage), so the wait counts at the loop top that
  // hold for the first pass hold for every pass.
  load_w(kbeg, cA, qA, sA);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dma_x_row(0, kbeg, j);
    dma_x_row(1, clampk(kbeg + 1), j);
  }
  __syncthreads();  // the 16-entry codebook (and this wave's loads have landed)
  pair_table_to_lds(tbl, lut16, tid);
  __syncthreads();  // pair table and X(0..1) visible to every wave
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float sc = dq_scale(qA[g], sA[g]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float f[8];
      lut8(cA[g][s], f);
      wc[g][s] = pack8(f, sc);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  load_w(clampk(kbeg + 1), cA, qA, sA);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma_x_row(2, clampk(kbeg + 2), j);
  __builtin_amdgcn_sched_barrier(0);
  read_x(0, 0, xa);

  // Substep S of a step: 16 slices, each one MFMA on (wc[.][S], XCUR) plus
  // at most one piece of each kind of side work, fenced off from the next
  // slice so the issue order stays interleaved:
  //  * slices 0..7 read X of the next substep (XNXT, ring stage RSTAGE,
  //    chunk RS) and look up one code byte of chunk S of the next step's
  //    codes CA (two codebook values, one 8-byte read of the pair table);
  //  * slices 8..15 scale and pack the pair looked up 8 slices earlier into
  //    wn[.][S];
  //  * EXTRA(i) adds the step's memory traffic and scale arithmetic.
#define QLORA_FWD_SUBSTEP(S, XCUR, XNXT, RSTAGE, RS, CA, EXTRA)                                        \
  {                                                                                                   \
    const unsigned char* xs_ = xring[RSTAGE] + ml * 128 + (((4 * h + (RS)) ^ sw) << 4);               \
    uint32_t pw_[2][4];                                                                               \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                                  \
      acc[i & 1][i >> 1] = mfma32(wc[i & 1][S], XCUR[i >> 1], acc[i & 1][i >> 1]);                    \
      if (i < 8) {                                                                                    \
        XNXT[i] = *reinterpret_cast<const bf16x8*>(xs_ + i * 4096);                                  \
        const int g_ = i >> 2, q_ = i & 3;                                                            \
        const float2 v_ = *reinterpret_cast<const float2*>(tbl + byte_x8(CA[g_][S], q_));            \
        fp[g_][2 * q_] = v_.x;                                                                        \
        fp[g_][2 * q_ + 1] = v_.y;                                                                    \
      } else {                                                                                        \
        const int g_ = (i - 8) >> 2, q_ = i & 3;                                                      \
        pw_[g_][q_] = pack_bf16x2(fp[g_][2 * q_] * sc[g_], fp[g_][2 * q_ + 1] * sc[g_]);              \
        if (q_ == 3) wn[g_][S] = as_bf16x8(pw_[g_][0], pw_[g_][1], pw_[g_][2], pw_[g_][3]);          \
      }                                                                                               \
      EXTRA;                                                                                          \
      __builtin_amdgcn_sched_barrier(0);                                                              \
    }                                                                                                 \
  }

  // One pipelined step; X(kb) is in ring stage ST, X(kb+1) in ST1, and
  // stage ST3 (X(kb-1)'s, read for the last time in step kb-1) receives
  // X(kb+3).  CA.. name the register set holding the codes of step kb+1
  // (decoded now), CB.. the set that receives the codes of step kb+2.  The
  // loop is unrolled by four so code sets (period 2) and stages (period 4)
  // are compile-time constants: no register copies (a copy would wait for
  // the load just issued) and statically distinct LDS objects.
  //  * substep 0 computes the scales of CA (slices 0, 2) and loads the codes
  //    of step kb+2 (slices 8..13);
  //  * substep 3 loads X(kb+3) into stage ST3 (slices 8..15).
  // The barrier before substep 3 publishes X(kb+1), loaded two steps ago:
  // each wave first waits for its own loads of that step (20 buffer
  // operations were issued after them) and leaves at most 8 LDS operations
  // in flight; after the barrier every wave is also done with step kb-1,
  // so stage ST3 is free.
#define QLORA_FWD_STEP(KB, ST, ST1, ST3, CA, QA, SA, CB, QB, SB)                                       \
  {                                                                                                    \
    const int kn2 = (KB) + 2 < nk ? (KB) + 2 : nk - 1; /* past the end: redundant, in bounds */        \
    const int kn3 = (KB) + 3 < nk ? (KB) + 3 : nk - 1;                                                 \
    float sc[2];                                                                                       \
    QLORA_FWD_SUBSTEP(0, xa, xb, ST, 1, CA, {                                                          \
      if (i == 0) sc[0] = dq_scale(QA[0], SA[0]);                                                      \
      if (i == 2) sc[1] = dq_scale(QA[1], SA[1]);                                                      \
      if (i >= 8 && i < 14) load_w_part(kn2, CB, QB, SB, i - 8);                                       \
    })                                                                                                 \
    QLORA_FWD_SUBSTEP(1, xb, xa, ST, 2, CA, {})                                                        \
    QLORA_FWD_SUBSTEP(2, xa, xb, ST, 3, CA, {})                                                        \
    asm volatile("s_waitcnt vmcnt(20) lgkmcnt(8)\n\ts_barrier" ::: "memory");                         \
    QLORA_FWD_SUBSTEP(3, xb, xa, ST1, 0, CA, {                                                         \
      if (i >= 8) dma_x_row(ST3, kn3, i - 8);                                                          \
    })                                                                                                 \
    _Pragma("unroll") for (int g = 0; g < 2; ++g) {                                                    \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) wc[g][s] = wn[g][s];                              \
    }                                                                                                  \
  }

  // Whole groups of four steps loop; the remainder runs once after the loop,
  // so the loop back-edge is reached from one path only and the wait counts
  // at its top stay exact.
  int kb = kbeg;
  for (; kb + 4 <= kend; kb += 4) {
    QLORA_FWD_STEP(kb, 0, 1, 3, cA, qA, sA, cB, qB, sB)
    QLORA_FWD_STEP(kb + 1, 1, 2, 0, cB, qB, sB, cA, qA, sA)
    QLORA_FWD_STEP(kb + 2, 2, 3, 1, cA, qA, sA, cB, qB, sB)
    QLORA_FWD_STEP(kb + 3, 3, 0, 2, cB, qB, sB, cA, qA, sA)
  }
  if (kb < kend) {
    QLORA_FWD_STEP(kb, 0, 1, 3, cA, qA, sA, cB, qB, sB)
    if (kb + 1 < kend) QLORA_FWD_STEP(kb + 1, 1, 2, 0, cB, qB, sB, cA, qA, sA)
    if (kb + 2 < kend) QLORA_FWD_STEP(kb + 2, 2, 3, 1, cA, qA, sA, cB, qB, sB)
  }
#undef QLORA_FWD_STEP
#undef QLORA_FWD_SUBSTEP

  // LoRA up-projection as two more K-steps of 64 j per pass: A operand =
  // B^T (rows n), B operand = the bf16 hi and lo rows of s XA (rows m), so
  // the fp32 XA keeps ~16 significant bits even where the adapter term
  // dominates Y.  Slice 0 carries it.  The B^T tile is built in LDS by
  // loading 8 rows j x 8 columns n per lane and transposing them in
  // registers; the hi / lo tiles are copied by buffer-to-LDS loads straight
  // into the swizzled X-stage layout.
  if (sidx == 0) {
    const int r = p.r;
    const rsrc_t rh = make_rsrc(P.XAh + m0 * p.RP, (T - m0) * p.RP * 2);
    const rsrc_t rl = make_rsrc(P.XAl + m0 * p.RP, (T - m0) * p.RP * 2);
    const int bjg = tid & 7, bng = tid >> 3;  // lane's 8 j and 8 n of the B tile
    const int64_t bn = n0 + 8 * bng;
    const int drow = lane >> 3, dphys = lane & 7;
    for (int jb = 0; jb < p.RP; jb += 64) {
      u32x4 brow[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = jb + 8 * bjg + i;
        brow[i] = (j < r && bn < N) ? *reinterpret_cast<const u32x4*>(P.B + (int64_t)j * N + bn)
                                    : u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();  // every wave is done with the stages
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + drow;
        const uint32_t off = (uint32_t)(row * p.RP * 2 + (jb + 8 * (dphys ^ ((row >> 1) & 7))) * 2);
        buf_load16_to_lds(rh, xring[1] + (64 * wave + 8 * i) * 128, off);
        buf_load16_to_lds(rl, xring[2] + (64 * wave + 8 * i) * 128, off);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_perm(brow[2 * q + 1][c >> 1], brow[2 * q][c >> 1], sel);
        const int row = 8 * bng + c;
        *reinterpret_cast<u32x4*>(xring[0] + row * 128 + ((bjg ^ ((row >> 1) & 7)) << 4)) = v;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 aop[2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
          aop[g] = *reinterpret_cast<const bf16x8*>(xring[0] + (64 * wave + 32 * g + ml) * 128 + (((4 * h + s) ^ sw) << 4));
        read_x(1, s, xa);
        read_x(2, s, xb);
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            acc[g][mi] = mfma32(aop[g], xa[mi], acc[g][mi]);
            acc[g][mi] = mfma32(aop[g], xb[mi], acc[g][mi]);
          }
      }
    }
  }

  if (it.S > 1) {
    __syncthreads();  // every wave is done with LDS; word 16 holds the ticket
    if (!splitk_combine(acc, p.slots + (int64_t)it.ordinal * it.S * kSplitSlotFloats, p.counters + it.ordinal,
                        p.counters + p.plan.nsplit() + it.ordinal,
                        it.S, sidx, reinterpret_cast<int*>(tbl + 2112), p.status))
      return;
  }

  // Y through LDS: D[n][m] of a 32x32 tile gives lane (ml, h) token
  // m = 32 mi + ml and the 4 features 8 q4 + 4h + (0..3), written as bf16
  // into [64 m][256 n] tiles (stage q holds token rows 64q .. 64q + 63)
  // whose 16-byte chunks are XOR-swizzled by the row (the 32 lanes of a
  // write land in 32 distinct chunks); then each 32 lanes store one whole
  // 512-byte row of Y.
  __syncthreads();  // every wave is done with the stages
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    unsigned char* const yst = xring[mi >> 1];
    const int row = 32 * (mi & 1) + ml;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 8 * wave + 4 * g + q4;
        const f32x16& a = acc[g][mi];
        *reinterpret_cast<uint2*>(yst + row * 512 + ((c ^ ml) << 4) + 8 * h) =
            make_uint2(pack_bf16x2(a[4 * q4 + 0], a[4 * q4 + 1]), pack_bf16x2(a[4 * q4 + 2], a[4 * q4 + 3]));
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int idx = 256 * i + tid, row = idx >> 5, c = idx & 31;  // row 0..255 = 64 * (i / 8) + ..
    const int64_t m = m0 + row, n = n0 + 8 * c;
    const u32x4 v = *reinterpret_cast<const u32x4*>(xring[i >> 3] + (row & 63) * 512 + ((c ^ (row & 31)) << 4));
    if (m < T && n < N) *reinterpret_cast<u32x4*>(P.Y + m * N + n) = v;  // N % 8 == 0: chunks whole
  }
}

SplitPlan fwd_plan(int64_t T, int64_t K, int64_t N, int batch) {
  return make_split_plan((int64_t)batch * ((N + kTileN - 1) / kTileN) * ((T + kTileM - 1) / kTileM), K / 64);
}

hipError_t launch_gemm_fwd(const FwdGemmParams& p0, const Codebook& cb, hipStream_t s) {
  FwdGemmParams p = p0;
  p.batch = 1;
  p.prob[0] = FwdGemmProblem{p.X, p.codes, p.q8, p.s2, p.B, p.XAh, p.XAl, p.Y};
  return launch_gemm_fwd_batched(p, cb, s);
}

hipError_t launch_gemm_fwd_batched(const FwdGemmParams& p0, const Codebook& cb, hipStream_t s) {
  FwdGemmParams p = p0;
  p.tiles_n = (int)((p.N + kTileN - 1) / kTileN);
  p.tiles_m = (int)((p.T + kTileM - 1) / kTileM);
  p.tiles_per = p.tiles_n * p.tiles_m;
  p.plan = fwd_plan(p.T, p.K, p.N, p.batch);
  {
    KernelTimer kt_("gemm_fwd_kernel", s);
    hipLaunchKernelGGL(gemm_fwd_kernel, dim3(8 * p.plan.items), dim3(256), 0, s, p, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
