// Launchers of the dequantize-GEMM / GEMV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "splitk.hpp"

namespace qlora {

// Same-shape problems of one batched GEMM launch (q/k/v, gate/up): their
// tiles are numbered problem-major and share one split plan.
constexpr int kGemmBatchMax = 4;
struct FwdGemmProblem {
  const uint16_t* X;     // [T,K] bf16
  const uint8_t* codes;  // [N*K/2]
  const uint8_t* q8;     // [N*K/64]
  const float* s2;       // [ceil(N*K/64/256)]
  const uint16_t* B;     // [r,N] bf16
  const uint16_t* XAh;   // [T,RP] bf16 hi part of s*XA
  const uint16_t* XAl;   // [T,RP] bf16 lo part
  uint16_t* Y;           // [T,N] bf16
};
struct DxGemmProblem {
  const uint16_t* dY;    // [T,N] bf16
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;     // [K,r] bf16
  const uint16_t* Gh;    // [T,RP] bf16 hi part of s*G
  const uint16_t* Gl;    // [T,RP] bf16 lo part
  uint16_t* dX;          // [T,K] bf16
};

struct FwdGemmParams {
  const uint16_t* X;     // [T,K] bf16
  const uint8_t* codes;  // [N*K/2]
  const uint8_t* q8;     // [N*K/64]
  const float* s2;       // [ceil(N*K/64/256)]
  const uint16_t* B;     // [r,N] bf16
  float* XA;             // [T,r] fp32 out (GEMV path: computed by the GEMV itself)
  const uint16_t* A;     // [K,r] bf16 (GEMV path)
  float* P;              // GEMV path: partials of XA, [nparts][T][RP]
  int nparts;            // GEMV path: their count (filled by the launcher)
  const uint16_t* XAh;   // [T,RP] bf16 hi part of s*XA, zero past r (GEMM path)
  const uint16_t* XAl;   // [T,RP] bf16 lo part
  uint16_t* Y;           // [T,N] bf16
  int64_t T, K, N;
  int r, RP;             // RP = r rounded up to 64
  float s;
  float* slots;          // split partials: nsplit * S * 65536 floats (S > 1)
  int* counters;         // 2 per split tile (tickets, then published counts), zero on entry, left zero
  int* status;           // the device's status word (set if a split wait ran out)
  SplitPlan plan;        // filled by the launcher
  int tiles_n, tiles_m;  // filled by the launcher
  FwdGemmProblem prob[kGemmBatchMax];  // the batch (filled by the launcher for a single problem)
  int batch, tiles_per;  // problems, tiles per problem
};

struct DxGemmParams {
  const uint16_t* dY;    // [T,N] bf16
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;     // [K,r] bf16
  const uint16_t* Gh;    // [T,RP] bf16 hi part of s*G (G = dY B^T), zero past r
  const uint16_t* Gl;    // [T,RP] bf16 lo part
  uint16_t* dX;          // [T,K] bf16
  int64_t T, K, N;
  int r, RP;            // RP = r rounded up to 64
  float* slots;          // split partials: nsplit * S * 65536 floats (S > 1)
  int* counters;         // 2 per split tile (tickets, then published counts), zero on entry, left zero
  int* status;           // the device's status word (set if a split wait ran out)
  SplitPlan plan;        // filled by the launcher
  int tiles_k, tiles_t;
  DxGemmProblem prob[kGemmBatchMax];   // the batch (filled by the launcher for a single problem)
  int batch, tiles_per;  // problems, tiles per problem
};

// Grid of the GEMV and the slices of its XA partials: partial b < nparts
// sums the contraction over [b ks, min(K, (b+1) ks)).
struct GemvPlan {
  int grid, nparts, ks;
};
GemvPlan gemv_plan(int64_t N, int64_t K, int64_t T, int32_t r);

// A group of small-token forwards served by one XA-partial launch and one
// GEMV launch (T <= 16, shared T, r and s).  The launcher fills nparts, ks,
// wg_begin and part_begin.
constexpr int kGemvGroupMax = 8;
struct GemvLinear {
  const uint16_t* X;     // [T,K] bf16
  const uint8_t* codes;  // [N*K/2]
  const uint8_t* q8;     // [N*K/64]
  const float* s2;       // [ceil(N*K/64/256)]
  const uint16_t* A;     // [K,r]
  const uint16_t* B;     // [r,N]
  uint16_t* Y;           // [T,N] out
  float* XA;             // [T,r] out
  float* P;              // XA partials [nparts][T][RP] (workspace)
  int64_t K, N;
  int nparts, ks;        // XA partial slices (each ks of K)
  int wg_begin;          // first GEMV workgroup of this linear
  int part_begin;        // first XA-partial workgroup of this linear
};
// NMAX: the capacity of L.  Launches of a single linear use NMAX = 1, so their
// kernel argument block is an eighth of the size.
template <int NMAX>
struct GemvGroupT {
  GemvLinear L[NMAX];
  int count;
  int T, r, RP;          // RP = r rounded up to 64
  float s;
};
using GemvGroup = GemvGroupT<kGemvGroupMax>;
hipError_t launch_gemv_group(GemvGroup g, const Codebook& cb, hipStream_t s);

hipError_t launch_gemm_fwd(const FwdGemmParams& p, const Codebook& cb, hipStream_t s);
// Batched launches: p.prob[0 .. p.batch) are filled by the caller (the
// single-problem pointers of p are ignored); shapes, r and s are shared.
hipError_t launch_gemm_fwd_batched(const FwdGemmParams& p, const Codebook& cb, hipStream_t s);
hipError_t launch_gemm_dx_batched(const DxGemmParams& p, const Codebook& cb, hipStream_t s);
hipError_t launch_gemv_fwd(const FwdGemmParams& p, const Codebook& cb, hipStream_t s);
hipError_t launch_gemm_dx(const DxGemmParams& p, const Codebook& cb, hipStream_t s);

// Work plans of the two GEMMs for a T x K x N problem (the workspaces are
// sized from these).
SplitPlan dx_plan(int64_t T, int64_t K, int64_t N, int batch = 1);
SplitPlan fwd_plan(int64_t T, int64_t K, int64_t N, int batch = 1);

}  // namespace qlora
