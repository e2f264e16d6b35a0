// Orchestration of the forward and backward passes of the frozen NF4 linear
// layer with a LoRA adapter: workspace layout, path choice and launch order.
//
// Forward  (Y = X W'^T + s (X A) B, XA = X A):
//   1. rowdot X A  -> chunk partials -> XA (fp32, also the caller's output)
//   2. T <= 16: dequant-GEMV;  T > 16: dequant-GEMM; both add s XA B in
//      their epilogue.
// Backward (G = dY B^T; dX = dY W' + s G A^T; dA = s X^T G; dB = s XA^T dY):
//   1. rowdot dY B^T -> G (fp32, workspace)
//   2. tokdot dY^T XA -> dB
//   3. dequant-GEMM dX with the s G A^T term in its epilogue
//   4. tokdot X^T G -> dA
// Every reduction is split into chunks whose partials are summed in a fixed
// order, so results are bitwise reproducible.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "lora.hpp"

namespace qlora {

namespace {
constexpr int64_t kGemvMaxT = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Chunk length along the contraction of a rowdot (X A or dY B^T): enough
// chunks to give ~256 workgroups, each at least 64 long.
int64_t row_chunk(int64_t T, int64_t L) {
  const int64_t tiles = cdiv(T, 64);
  const int64_t target = cdiv(256, tiles);
  int64_t lc = cdiv(cdiv(L, target), 64) * 64;
  return lc < 64 ? 64 : lc;
}

// Token chunk of a tokdot (X^T G or dY^T XA): ~256 workgroups, >= 32 tokens.
int64_t tok_chunk(int64_t T, int64_t C) {
  const int64_t tiles = cdiv(C, 64);
  const int64_t target = cdiv(256, tiles);
  int64_t tc = cdiv(cdiv(T, target), 32) * 32;
  return tc < 32 ? 32 : tc;
}
}  // namespace

size_t fwd_workspace_bytes(int64_t T, int64_t K, int64_t /*N*/, int32_t r) {
  if (T <= 0) return 0;
  const int64_t lc = row_chunk(T, K);
  return align256((size_t)cdiv(K, lc) * T * r * sizeof(float));
}

size_t bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (T <= 0) return 0;
  const size_t pg = align256((size_t)cdiv(N, row_chunk(T, N)) * T * r * sizeof(float));
  const size_t g = align256((size_t)T * r * sizeof(float));
  const size_t pdb = (size_t)cdiv(T, tok_chunk(T, N)) * N * r * sizeof(float);
  const size_t pda = (size_t)cdiv(T, tok_chunk(T, K)) * K * r * sizeof(float);
  return pg + g + align256(pdb > pda ? pdb : pda);
}

hipError_t launch_linear_fwd(const LinearArgs& a, const Codebook& cb, const uint16_t* X, uint16_t* Y, float* XA,
                             void* ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  float* P = reinterpret_cast<float*>(ws);
  hipError_t e = launch_rowdot(X, a.A, /*v_kmajor=*/true, P, XA, a.T, a.K, a.r, row_chunk(a.T, a.K), s);
  if (e != hipSuccess) return e;
  FwdGemmParams p{};
  p.X = X;
  p.codes = a.codes;
  p.q8 = a.q8;
  p.s2 = a.s2;
  p.B = a.B;
  p.XA = XA;
  p.Y = Y;
  p.T = a.T;
  p.K = a.K;
  p.N = a.N;
  p.r = a.r;
  p.s = a.s;
  return a.T <= kGemvMaxT ? launch_gemv_fwd(p, cb, s) : launch_gemm_fwd(p, cb, s);
}

hipError_t launch_linear_bwd(const LinearArgs& a, const Codebook& cb, const uint16_t* dY, const uint16_t* X,
                             const float* XA, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, hipStream_t s) {
  if (a.T == 0) {
    hipError_t e = launch_zero_u16(dA, a.K * a.r, s);
    if (e != hipSuccess) return e;
    return launch_zero_u16(dB, (int64_t)a.r * a.N, s);
  }
  char* w = reinterpret_cast<char*>(ws);
  const int64_t lcg = row_chunk(a.T, a.N);
  float* Pg = reinterpret_cast<float*>(w);
  w += align256((size_t)cdiv(a.N, lcg) * a.T * a.r * sizeof(float));
  float* G = reinterpret_cast<float*>(w);
  w += align256((size_t)a.T * a.r * sizeof(float));
  float* Ptok = reinterpret_cast<float*>(w);

  hipError_t e = launch_rowdot(dY, a.B, /*v_kmajor=*/false, Pg, G, a.T, a.N, a.r, lcg, s);
  if (e != hipSuccess) return e;
  e = launch_tokdot(dY, XA, Ptok, dB, a.T, a.N, a.r, tok_chunk(a.T, a.N), a.s, /*transpose=*/true, s);
  if (e != hipSuccess) return e;
  DxGemmParams p{};
  p.dY = dY;
  p.codes = a.codes;
  p.q8 = a.q8;
  p.s2 = a.s2;
  p.A = a.A;
  p.G = G;
  p.dX = dX;
  p.T = a.T;
  p.K = a.K;
  p.N = a.N;
  p.r = a.r;
  p.s = a.s;
  e = launch_gemm_dx(p, cb, s);
  if (e != hipSuccess) return e;
  return launch_tokdot(X, G, Ptok, dA, a.T, a.K, a.r, tok_chunk(a.T, a.K), a.s, /*transpose=*/false, s);
}

}  // namespace qlora
