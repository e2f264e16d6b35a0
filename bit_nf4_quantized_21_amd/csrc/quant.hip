// Blockwise 4-bit quantization, double quantization and dequantization
// kernels for gfx950.
//
// NF4 and double quantization are items (a) and (b) of the QLoRA abstract
// ("QLoRA: Efficient Finetuning of Quantized LLMs"); Int4 and FP4 are the
// 4-bit types the pages compare NF4 with (news write-up, innovations list).
// The block sizes (64 and 256), the 8-bit constant format, the decode tables
// and the low-nibble-first packing are the readings documented in
// include/qlora.h.  Every type is quantized by the same rule: the code of the
// type's level nearest to w/absmax in exact arithmetic.
//
// A 64-weight block belongs to 16 lanes (one vector load per lane, a 4-step
// DPP row max for the absmax); each 16-lane group takes four blocks with
// their loads issued together.  Codes are decided exactly with one fp64
// product and compare per weight against the boundary of the weight's bin.
// With fp32 sources the kernels run near the HBM stream rate; with bf16
// sources the per-weight decision work bounds them.
// The double quantizer gives each group of 256 constants to one wavefront;
// the fused quantizer gives each group of 256 blocks to one workgroup and
// keeps the absmax values on chip.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "common.hpp"
#include "timing.hpp"
#include "kernels.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// Quantize: W[n] fp32 or bf16 -> codes[n/2], absmax[ceil(n/64)].
// ---------------------------------------------------------------------------

// Each 16-lane group quantizes kQGroupBlocks consecutive blocks; the loads of
// all of them are issued before any is used, so a wave keeps 4 KiB (fp32) or
// 2 KiB (bf16) of the weight stream in flight.  bf16 weights keep the same
// grid (8 blocks per group, half the waves, measured 13 % slower).
constexpr int kQGroupBlocks = 4;

// Four consecutive weights from e0 as fp32; zero past n.  A bf16 weight
// widens to fp32 exactly (its bits are the upper half of the fp32 word), so
// every decision below is the one taken for the same value given as fp32.
__device__ __forceinline__ void load_weights4(const float* __restrict__ W, int64_t n, int64_t e0, float (&v)[4]) {
  if (e0 + 4 <= n) {
    const float4 x = *reinterpret_cast<const float4*>(W + e0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < n) ? W[e0 + i] : 0.0f;
  }
}
__device__ __forceinline__ void load_weights4(const uint16_t* __restrict__ W, int64_t n, int64_t e0,
                                              float (&v)[4]) {
  if (e0 + 4 <= n) {
    const uint2 x = *reinterpret_cast<const uint2*>(W + e0);
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < n) ? __uint_as_float((uint32_t)W[e0 + i] << 16) : 0.0f;
  }
}

// Uniform bins of w / absmax over [-1, 1]: the host picks a count between
// kBinsMin and kBinsMax (128 first) whose bins separate the type's
// boundaries.
constexpr int kBinsMin = 96, kBinsMax = 160;
// Blocks whose absmax lies outside [kTinyAbsmax, kHugeAbsmax] take the exact
// scan: there 1/absmax (or its product with nbins/2) would leave the normal
// fp32 range and the bin estimate would lose its accuracy.
constexpr float kTinyAbsmax = 1e-30f;
constexpr float kHugeAbsmax = 0x1p120f;

// Exact scan: level = #{j : w > absmax * m_j} over the type's boundaries
// (absmax * m_j is exact in fp64; +inf boundaries never count).
__device__ __forceinline__ uint32_t scan_code(float w, double a64, const Midpoints& mp) {
  const double w64 = (double)w;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (w64 > a64 * mp.m[j]) ? 1u : 0u;
  return a64 == 0.0 ? mp.zero_code : level_code(mp, c);
}

// Bin tables of a type: every bin of width 2/nbins holds at most one level
// boundary, none within 1e-5 of a bin edge (checked on the host before the
// tables are built), so the bin of the fp32 estimate of w / absmax (error
// below 1e-6) contains its true position or is a neighbour separated from it
// by no boundary.  Entry b is one fp64 word: the bin's boundary (2.0, above
// every |w| / absmax, when it has none), whose low 8 mantissa bits, zero in
// every boundary (they have at most 29 significant bits), carry the code
// below the boundary (bits 0..3) and the code above it (bits 4..7); one 8-byte
// LDS read per weight gives both.  The host builds the tables once per launch
// and passes them by value; each workgroup copies them into LDS.
struct BinEntry {
  uint32_t lo, hi;  // the fp64 word, low dword first
};
struct BinTables {
  BinEntry e[kBinsMax];
  int nbins;
};
__device__ __forceinline__ void bin_tables_to_lds(BinTables& t, const BinTables& src) {
  if ((int)threadIdx.x < src.nbins) t.e[threadIdx.x] = src.e[threadIdx.x];
}

// a = max(a, a of the lane that the DPP control names), within rows of 16
// lanes.  One v_max_f32 with a DPP source (the builtin form adds a NaN
// canonicalization per step); s_nop 1 covers the wait states between a VALU
// write of a and its DPP read.
#define QLORA_ROW_MAX_STEP(a, ctrl) \
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf" : "=v"(a) : "v"(a))

// Maximum over the 16 lanes of a DPP row, on every lane of the row: swaps
// within quads (quad_perm [1,0,3,2], then [2,3,0,1]), then the half-row and
// the row mirrors.  VALU only (a cross-lane shuffle would go through the LDS
// crossbar); the maximum of the same 16 values, so the same bits.
__device__ __forceinline__ float row16_max(float a) {
  QLORA_ROW_MAX_STEP(a, "quad_perm:[1,0,3,2]");
  QLORA_ROW_MAX_STEP(a, "quad_perm:[2,3,0,1]");
  QLORA_ROW_MAX_STEP(a, "row_half_mirror");
  QLORA_ROW_MAX_STEP(a, "row_mirror");
  return a;
}
#undef QLORA_ROW_MAX_STEP

// Quantizes the block held by a 16-lane group (lane l16 holds elements
// 4 l16 .. 4 l16 + 3 in v): returns the 4 codes packed low nibble first and
// the block's absmax in *amax (on every lane of the group).
__device__ __forceinline__ uint32_t quantize_block(const float (&v)[4], const Midpoints& mp, const BinTables& bt,
                                                   int nbins, float* amax) {
  const float a = row16_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  *amax = a;
  const double a64 = (double)a;
  uint32_t c[4];
  if (a < kTinyAbsmax || a > kHugeAbsmax) {  // uniform per 16-lane group; absmax 0 -> the zero code
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = scan_code(v[i], a64, mp);
  } else {
    // Bin position x = (w / absmax + 1) nbins / 2 as one fma; x > -1 since
    // |w| <= absmax, so truncation never goes below bin 0, and w = absmax
    // reaches x = nbins, the last bin's upper edge.
    const float half = 0.5f * (float)nbins, ih = __builtin_amdgcn_rcpf(a) * half;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int b = (int)__builtin_fmaf(v[i], ih, half);
      b = b < nbins - 1 ? b : nbins - 1;
      const BinEntry e = bt.e[b];
      const double thr = __hiloint2double((int)e.hi, (int)(e.lo & ~0xFFu));
      c[i] = (e.lo >> (((double)v[i] > a64 * thr) ? 4 : 0)) & 15u;
    }
  }
  return c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12);
}

// Stores the 4 codes of elements e0 .. e0 + 3 (n is even: pairs are whole).
__device__ __forceinline__ void store_codes4(uint8_t* __restrict__ codes, int64_t n, int64_t e0, uint32_t packed) {
  if (e0 + 4 <= n) {
    *reinterpret_cast<uint16_t*>(codes + e0 / 2) = (uint16_t)packed;
  } else {
    if (e0 < n) codes[e0 / 2] = (uint8_t)(packed & 0xFF);
    if (e0 + 2 < n) codes[e0 / 2 + 1] = (uint8_t)(packed >> 8);
  }
}

template <typename T>
__device__ __forceinline__ void quantize_blocks(const T* __restrict__ W, int64_t n, uint8_t* __restrict__ codes,
                                                float* __restrict__ absmax, const Midpoints& mp,
                                                const BinTables& bins) {
  __shared__ BinTables bt;
  const int nbins = bins.nbins;
  bin_tables_to_lds(bt, bins);
  __syncthreads();
  const int64_t nb = (n + kBlock - 1) / kBlock;
  constexpr int G = kQGroupBlocks;
  const int64_t blk0 = ((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) * G;
  const int l16 = threadIdx.x & 15;
  if (blk0 >= nb) return;  // whole 16-lane groups leave together (after the barrier)
  float v[G][4];
  if ((blk0 + G) * kBlock <= n) {
    // Every block of the group is whole (all but the last groups): plain
    // vector loads and stores, no per-element range checks.
#pragma unroll
    for (int g = 0; g < G; ++g) load_weights4(W, INT64_MAX, (blk0 + g) * kBlock + l16 * 4, v[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a;
      const uint32_t packed = quantize_block(v[g], mp, bt, nbins, &a);
      if (l16 == 0) absmax[blk0 + g] = a;
      store_codes4(codes, INT64_MAX, (blk0 + g) * kBlock + l16 * 4, packed);
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) load_weights4(W, n, (blk0 + g) * kBlock + l16 * 4, v[g]);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t blk = blk0 + g;
    if (blk >= nb) break;  // uniform per 16-lane group
    float a;
    const uint32_t packed = quantize_block(v[g], mp, bt, nbins, &a);
    if (l16 == 0) absmax[blk] = a;
    store_codes4(codes, n, blk * kBlock + l16 * 4, packed);
  }
}

// One kernel per weight type and decision flavour, so that traces tell them
// apart.
__global__ __launch_bounds__(256) void quantize_nf4_kernel(const float* __restrict__ W, int64_t n,
                                                           uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                           Midpoints mp, BinTables bins) {
  quantize_blocks<float>(W, n, codes, absmax, mp, bins);
}
__global__ __launch_bounds__(256) void quantize_nf4_bf16_kernel(const uint16_t* __restrict__ W, int64_t n,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ absmax, Midpoints mp,
                                                                BinTables bins) {
  quantize_blocks<uint16_t>(W, n, codes, absmax, mp, bins);
}
// ---------------------------------------------------------------------------
// Fused quantize + double quant: W[n] -> codes[n/2], q8[nb], s2[ceil(nb/256)].
// One workgroup per group of 256 blocks (16384 weights): four passes of 64
// blocks quantize the weights as above and keep each block's fp32 absmax in
// LDS; then thread t turns absmax t into its 8-bit code against the group's
// maximum.  The absmax values never travel through memory.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t q8_code(float c, double s2d, double scale);

template <typename T>
__device__ __forceinline__ void quantize_dq_group(const T* __restrict__ W, int64_t n, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ q8, float* __restrict__ s2,
                                                  const Midpoints& mp, const BinTables& bins) {
  __shared__ BinTables bt;
  __shared__ float s_amax[kBlock2];
  __shared__ float s_wmax[4];
  const int nbins = bins.nbins;
  bin_tables_to_lds(bt, bins);
  __syncthreads();
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t gblk = (int64_t)blockIdx.x * kBlock2;  // first block of the group
  const int l16 = threadIdx.x & 15, lg = threadIdx.x >> 4;
  constexpr int G = kQGroupBlocks;
  // The four passes of 64 blocks; FULL: all 256 blocks of the group are
  // whole (every group but the last), so loads and stores need no range
  // checks.
  auto passes = [&](auto full) {
    constexpr bool FULL = decltype(full)::value;
    constexpr int kPasses = kBlock2 / (16 * G);
    auto load_pass = [&](int pass, float (&v)[G][4]) {
      const int local0 = pass * 16 * G + lg * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t blk = gblk + local0 + g;
        if (FULL) load_weights4(W, INT64_MAX, blk * kBlock + l16 * 4, v[g]);
        else if (blk < nb) load_weights4(W, n, blk * kBlock + l16 * 4, v[g]);
        else v[g][0] = v[g][1] = v[g][2] = v[g][3] = 0.0f;
      }
    };
    // The next pass's weights are loading while this pass is decided.
    float vb[2][G][4];
    load_pass(0, vb[0]);
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int local0 = pass * 16 * G + lg * G;  // block of the group, 0..255
      if (pass + 1 < kPasses) load_pass(pass + 1, vb[(pass + 1) & 1]);
      float (&v)[G][4] = vb[pass & 1];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t blk = gblk + local0 + g;
        float a;
        const uint32_t packed = quantize_block(v[g], mp, bt, nbins, &a);  // every lane group takes part
        if (l16 == 0) s_amax[local0 + g] = a;                                // 0 past the last block
        if (FULL) store_codes4(codes, INT64_MAX, blk * kBlock + l16 * 4, packed);
        else if (blk < nb) store_codes4(codes, n, blk * kBlock + l16 * 4, packed);
      }
    }
  };
  if ((gblk + kBlock2) * kBlock <= n) passes(std::true_type{});  // uniform over the workgroup
  else passes(std::false_type{});
  __syncthreads();
  // s2 = the group's maximum absmax (exact fp32; the zeros past the last
  // block never raise it), then q8 of block t.
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float c = s_amax[t];
  float m = c;
#pragma unroll
  for (int off = 32; off; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) s_wmax[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  if (t == 0) s2[blockIdx.x] = m;
  const double s2d = (double)m;
  const uint32_t q = m > 0.0f ? q8_code(c, s2d, 255.0 / s2d) : 0u;
  if (gblk + t < nb) q8[gblk + t] = (uint8_t)q;
}

__global__ __launch_bounds__(256) void quantize_dq_kernel(const float* __restrict__ W, int64_t n,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ q8,
                                                          float* __restrict__ s2, Midpoints mp, BinTables bins) {
  quantize_dq_group<float>(W, n, codes, q8, s2, mp, bins);
}
__global__ __launch_bounds__(256) void quantize_dq_bf16_kernel(const uint16_t* __restrict__ W, int64_t n,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ q8, float* __restrict__ s2,
                                                               Midpoints mp, BinTables bins) {
  quantize_dq_group<uint16_t>(W, n, codes, q8, s2, mp, bins);
}

// ---------------------------------------------------------------------------
// Double quant: absmax[nb] -> q8[nb], s2[ceil(nb/256)].  One wave per group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t q8_code(float c, double s2d, double scale) {
  // Nearest integer to 255*c/s2, ties to even.  k0 = floor(c*255/s2) is
  // within one of the answer; 510*c and (2*k0+1)*s2 are exact in fp64 and
  // decide between k0 and k0+1.
  double cd = (double)c;
  double k0 = floor(cd * scale);
  double lhs = 510.0 * cd, rhs = (2.0 * k0 + 1.0) * s2d;
  int64_t k = (int64_t)k0;
  if (lhs > rhs || (lhs == rhs && (k & 1))) k += 1;
  k = k < 0 ? 0 : (k > 255 ? 255 : k);
  return (uint32_t)k;
}

__global__ __launch_bounds__(256) void double_quant_kernel(const float* __restrict__ absmax, int64_t nb,
                                                           uint8_t* __restrict__ q8, float* __restrict__ s2) {
  const int64_t ng = (nb + kBlock2 - 1) / kBlock2;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= ng) return;  // whole waves leave together
  const int64_t e0 = g * kBlock2 + lane * 4;
  const bool full = e0 + 4 <= nb;
  float v[4];
  if (full) {
    float4 x = *reinterpret_cast<const float4*>(absmax + e0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (e0 + i < nb) ? absmax[e0 + i] : 0.0f;
  }
  float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
  for (int off = 32; off; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) s2[g] = m;
  const double s2d = (double)m;
  const double scale = m > 0.0f ? 255.0 / s2d : 0.0;
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = m > 0.0f ? q8_code(v[i], s2d, scale) : 0u;
  if (full) {
    *reinterpret_cast<uint32_t*>(q8 + e0) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i < nb) q8[e0 + i] = (uint8_t)q[i];
  }
}

// ---------------------------------------------------------------------------
// Dequantize (support): 8 weights per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ q8,
                                                         const float* __restrict__ s2, int64_t n,
                                                         int out_bf16, void* __restrict__ out, Codebook cb) {
  __shared__ __align__(16) float lut[16];
  codebook_to_lds(lut, cb, threadIdx.x);
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= n) return;
  const int64_t b = e0 / kBlock;
  const float sc = dq_scale(q8[b], s2[b / kBlock2]);
  float w[8];
  if (e0 + 8 <= n) {
    uint32_t x = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = lut[(x >> (4 * i)) & 15] * sc;
    if (out_bf16) {
      u32x4 o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                 pack_bf16x2(w[6], w[7])};
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e0) = o;
    } else {
      float* o = reinterpret_cast<float*>(out) + e0;
      *reinterpret_cast<float4*>(o) = make_float4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(w[4], w[5], w[6], w[7]);
    }
  } else {
    for (int64_t e = e0; e < n; e += 2) {
      uint32_t x = codes[e / 2];
      float lo = lut[x & 15] * sc, hi = lut[x >> 4] * sc;
      if (out_bf16) {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + e) = pack_bf16x2(lo, hi);
      } else {
        reinterpret_cast<float*>(out)[e] = lo;
        reinterpret_cast<float*>(out)[e + 1] = hi;
      }
    }
  }
}

// ---------------------------------------------------------------------------
namespace {
// nbins uniform bins can be used when each holds at most one boundary of the
// type and none lies within 1e-5 of a bin edge.
bool bins_separate(const Midpoints& mp, int nbins) {
  for (int b = 0; b < nbins; ++b) {
    const double lo = -1.0 + b * (2.0 / nbins), hi = lo + 2.0 / nbins;
    int inside = 0;
    for (int j = 0; j < 15; ++j) {
      if (!std::isfinite(mp.m[j])) continue;
      if (mp.m[j] >= lo && mp.m[j] < hi) ++inside;
      if (std::fabs(mp.m[j] - lo) < 1e-5 || std::fabs(mp.m[j] - hi) < 1e-5) return false;
    }
    if (inside > 1) return false;
  }
  return true;
}

// The bin count for a type: 128, else the nearest count in range that
// separates its boundaries (INT4's and FP4's fall on edges of 128 bins;
// 127 separates NF4, INT4 and FP4 alike); 0 when none does.  The launchers
// refuse a call whose type has no bin count or a boundary with low mantissa
// bits set (no shipped type comes to either).
int choose_bins(const Midpoints& mp) {
  for (int d = 0; d <= kBinsMax - kBinsMin; ++d) {
    const int lo = 128 - d, hi = 128 + d;
    if (lo >= kBinsMin && bins_separate(mp, lo)) return lo;
    if (hi <= kBinsMax && bins_separate(mp, hi)) return hi;
  }
  return 0;
}

// The tables of nbins bins (the rule is stated at BinTables).
BinTables make_bins(const Midpoints& mp, int nbins) {
  BinTables t{};
  t.nbins = nbins;
  for (int b = 0; b < nbins; ++b) {
    const double lo = -1.0 + b * (2.0 / nbins), hi = lo + 2.0 / nbins;
    uint32_t cnt = 0;
    double thr = 2.0;
    for (int j = 0; j < 15; ++j) {
      if (mp.m[j] < lo) cnt += 1;
      else if (mp.m[j] < hi) thr = mp.m[j];
    }
    uint64_t bits;
    std::memcpy(&bits, &thr, sizeof bits);
    if (bits & 0xFFu) return BinTables{};  // a boundary using its low mantissa bits: refused (nbins = 0)
    bits |= level_code(mp, cnt) | (level_code(mp, cnt + 1 < 16 ? cnt + 1 : 15) << 4);
    t.e[b].lo = (uint32_t)bits;
    t.e[b].hi = (uint32_t)(bits >> 32);
  }
  return t;
}

template <typename T>
hipError_t launch_quantize_t(void (*binned_kernel)(const T*, int64_t, uint8_t*, float*, Midpoints, BinTables),
                             const T* W,
                             int64_t n, uint8_t* codes, float* absmax, const Midpoints& mp, const char* name,
                             hipStream_t s) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  constexpr int G = kQGroupBlocks;
  const int64_t grid = (nb + 16 * G - 1) / (16 * G);
  const int nbins = choose_bins(mp);
  const BinTables bins = nbins ? make_bins(mp, nbins) : BinTables{};
  if (bins.nbins == 0) return hipErrorInvalidValue;
  {
    KernelTimer kt_(name, s);
    hipLaunchKernelGGL(binned_kernel, dim3((unsigned)grid), dim3(256), 0, s, W, n, codes, absmax, mp, bins);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_dq_t(void (*binned_kernel)(const T*, int64_t, uint8_t*, uint8_t*, float*, Midpoints,
                                                      BinTables),
                                const T* W, int64_t n, uint8_t* codes, uint8_t* q8, float* s2, const Midpoints& mp,
                                const char* name, hipStream_t s) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t grid = (nb + kBlock2 - 1) / kBlock2;
  const int nbins = choose_bins(mp);
  const BinTables bins = nbins ? make_bins(mp, nbins) : BinTables{};
  if (bins.nbins == 0) return hipErrorInvalidValue;
  {
    KernelTimer kt_(name, s);
    hipLaunchKernelGGL(binned_kernel, dim3((unsigned)grid), dim3(256), 0, s, W, n, codes, q8, s2, mp, bins);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize_nf4(const float* W, int64_t n, uint8_t* codes, float* absmax, const Midpoints& mp,
                               hipStream_t s) {
  return launch_quantize_t(quantize_nf4_kernel, W, n, codes, absmax, mp, "quantize_nf4_kernel", s);
}

hipError_t launch_quantize_nf4_bf16(const uint16_t* W, int64_t n, uint8_t* codes, float* absmax,
                                    const Midpoints& mp, hipStream_t s) {
  return launch_quantize_t(quantize_nf4_bf16_kernel, W, n, codes, absmax, mp, "quantize_nf4_bf16_kernel", s);
}

hipError_t launch_quantize_dq(const void* W, bool bf16, int64_t n, uint8_t* codes, uint8_t* q8, float* s2,
                              const Midpoints& mp, hipStream_t s) {
  if (bf16)
    return launch_quantize_dq_t(quantize_dq_bf16_kernel, static_cast<const uint16_t*>(W), n, codes, q8, s2, mp,
                                "quantize_dq_bf16_kernel", s);
  return launch_quantize_dq_t(quantize_dq_kernel, static_cast<const float*>(W), n, codes, q8, s2, mp,
                              "quantize_dq_kernel", s);
}

hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* q8, float* s2, hipStream_t s) {
  const int64_t ng = (nb + kBlock2 - 1) / kBlock2;
  const int64_t grid = (ng + 3) / 4;
  {
    KernelTimer kt_("double_quant_kernel", s);
    hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, absmax, nb, q8, s2);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                             int out_bf16, void* out, const Codebook& cb, hipStream_t s) {
  const int64_t groups = (n + 7) / 8;
  const int64_t grid = (groups + 255) / 256;
  {
    KernelTimer kt_("dequantize_kernel", s);
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, q8, s2, n, out_bf16,
                     out, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
