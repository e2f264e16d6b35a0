// Orchestration of the forward and backward passes of the frozen NF4 linear
// layer with a LoRA adapter: workspace layout, path choice and launch order.
//
// Forward  (Y = X W'^T + s (X A) B, XA = X A; XA is also the caller's output):
//   T <= 16: 1. XA partials over slices of K (MFMA)
//            2. dequant-GEMV, summing the partials into XA and adding s XA B
//               in its epilogue.
//   T > 16:  1. rowdot X A -> chunk partials -> XA
//            2. dequant-GEMM, adding s XA B in its epilogue.
// Backward (G = dY B^T; dX = dY W' + s G A^T; dA = s X^T G; dB = s XA^T dY):
//   1. rowdot dY B^T -> G, kept as bf16 hi / lo parts: rows of s G for the
//      dX GEMM, tokdot planes of G and of XA
//   2. tokdots dY^T XA -> dB and X^T G -> dA, one launch
//   3. dequant-GEMM dX with the s G A^T term in its epilogue
// Every reduction is split into chunks whose partials are summed in a fixed
// order, so results are bitwise reproducible.
#include "common.hpp"
#include "device_state.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "lora.hpp"
#include "splitk.hpp"

namespace qlora {

namespace {
constexpr int64_t kGemvMaxT = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
int64_t rpad(int32_t r) { return round_up(r, 64); }

// Chunk of the contraction of a rowdot (X A or dY B^T): about 256
// workgroups of 64 rows each, chunks a multiple of 128 long.
int64_t row_chunk(int64_t T, int64_t L) {
  const int64_t tiles = cdiv(T, 64);
  int64_t nc = cdiv(256, tiles);
  const int64_t maxc = cdiv(L, 128);
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  return round_up(cdiv(L, nc), 128);
}

// Token chunk of a tokdot (X^T G or dY^T XA): about 256 workgroups of 64
// columns each, chunks a multiple of 128 tokens.
int64_t tok_chunk(int64_t T, int64_t C) {
  const int64_t tiles = cdiv(C, 64);
  int64_t nc = cdiv(256, tiles);
  const int64_t maxc = cdiv(T, 128);
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  return round_up(cdiv(T, nc), 128);
}

// Backward workspace regions, each 256-byte aligned.
struct BwdLayout {
  size_t pg, g, planes, ptok_b, ptok_a, slots, counters, total;
};
BwdLayout bwd_layout(int64_t T, int64_t K, int64_t N, int32_t r) {
  BwdLayout l{};
  const int64_t RP = rpad(r), TP = round_up(T, 64);
  l.pg = align256((size_t)cdiv(N, row_chunk(T, N)) * T * RP * sizeof(float));
  l.g = align256((size_t)T * RP * sizeof(uint16_t));
  l.planes = align256((size_t)RP * TP * sizeof(uint16_t));
  const size_t pdb = (size_t)cdiv(T, tok_chunk(T, N)) * RP * N * sizeof(float);
  const size_t pda = (size_t)cdiv(T, tok_chunk(T, K)) * RP * K * sizeof(float);
  l.ptok_b = align256(pdb);
  l.ptok_a = align256(pda);
  const SplitPlan dp = dx_plan(T, K, N);
  l.slots = dp.S > 1 ? align256((size_t)dp.nsplit() * dp.S * kSplitSlotFloats * sizeof(float)) : 0;
  l.counters = align256((size_t)(dp.nsplit() > 0 ? 2 * dp.nsplit() : 1) * sizeof(int));
  l.total = l.pg + 2 * l.g + 4 * l.planes + l.ptok_b + l.ptok_a + l.slots + l.counters;
  return l;
}
}  // namespace

// Forward workspace: GEMV path, the XA partials; GEMM path,
// rowdot partials, bf16 parts of s XA, split partials and tile counters.
struct FwdLayout {
  size_t p, xah, slots, counters, total;
  SplitPlan g;
};
FwdLayout fwd_layout(int64_t T, int64_t K, int64_t N, int32_t r) {
  FwdLayout l{};
  if (T <= kGemvMaxT) {
    l.p = align256((size_t)gemv_plan(N, K, T, r).nparts * T * rpad(r) * sizeof(float));
  } else {
    l.p = align256((size_t)cdiv(K, row_chunk(T, K)) * T * rpad(r) * sizeof(float));
    l.xah = align256((size_t)T * rpad(r) * sizeof(uint16_t));
    l.g = fwd_plan(T, K, N);
    l.slots = l.g.S > 1 ? align256((size_t)l.g.nsplit() * l.g.S * kSplitSlotFloats * sizeof(float)) : 0;
    l.counters = align256((size_t)(l.g.nsplit() > 0 ? 2 * l.g.nsplit() : 1) * sizeof(int));
  }
  l.total = l.p + 2 * l.xah + l.slots + l.counters;
  return l;
}

// Every kernel addresses its operands through buffer views whose size and
// offsets are 32-bit (at most 2^31 - 1 bytes), so a problem is accepted only
// if each operand and each workspace region fits one view.
bool linear_views_fit(int64_t T, int64_t K, int64_t N, int32_t r) {
  const int64_t lim = 0x7FFFFFFF;
  const int64_t RP = rpad(r);
  if (N * K / 2 > lim || T * K * 2 > lim || T * N * 2 > lim) return false;
  if (K * RP * 2 > lim || RP * N * 2 > lim || T * RP * 4 > lim) return false;
  if (T <= 0) return true;
  const FwdLayout f = fwd_layout(T, K, N, r);
  const BwdLayout b = bwd_layout(T, K, N, r);
  const size_t regions[] = {f.p, f.xah, f.slots, b.pg, b.g, b.planes, b.ptok_b, b.ptok_a, b.slots};
  for (size_t x : regions)
    if (x > (size_t)lim) return false;
  return true;
}

size_t fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (T <= 0) return 0;
  return fwd_layout(T, K, N, r).total;
}

size_t bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (T <= 0) return 0;
  return bwd_layout(T, K, N, r).total;
}

hipError_t launch_linear_fwd(const LinearArgs& a, const Codebook& cb, const uint16_t* X, uint16_t* Y, float* XA,
                             void* ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const FwdLayout l = fwd_layout(a.T, a.K, a.N, a.r);
  char* w = reinterpret_cast<char*>(ws);
  float* P = reinterpret_cast<float*>(w);
  uint16_t* XAh = reinterpret_cast<uint16_t*>(w + l.p);
  uint16_t* XAl = reinterpret_cast<uint16_t*>(w + l.p + l.xah);
  char* w2 = w + l.p + 2 * l.xah;
  if (a.T > kGemvMaxT) {
    RowdotOut o{};
    o.f32 = XA;
    o.row_hi = XAh;  // s XA as bf16 hi / lo rows for the GEMM's adapter steps
    o.row_lo = XAl;
    o.scale_row = a.s;
    o.zero = reinterpret_cast<int*>(w2 + l.slots);  // the GEMM's split tickets
    o.nzero = 2 * l.g.nsplit();
    hipError_t e = launch_rowdot(X, a.A, /*v_lr=*/true, P, o, a.T, a.K, a.r, row_chunk(a.T, a.K), s);
    if (e != hipSuccess) return e;
  }
  FwdGemmParams p{};
  hipError_t es = hipSuccess;
  p.status = status_word(&es);
  if (!p.status) return es;
  p.X = X;
  p.codes = a.codes;
  p.q8 = a.q8;
  p.s2 = a.s2;
  p.A = a.A;
  p.B = a.B;
  p.XA = XA;
  p.P = P;
  p.Y = Y;
  p.T = a.T;
  p.K = a.K;
  p.N = a.N;
  p.r = a.r;
  p.s = a.s;
  p.XAh = XAh;
  p.XAl = XAl;
  p.RP = (int)rpad(a.r);
  p.slots = reinterpret_cast<float*>(w2);
  p.counters = reinterpret_cast<int*>(w2 + l.slots);
  return a.T <= kGemvMaxT ? launch_gemv_fwd(p, cb, s) : launch_gemm_fwd(p, cb, s);
}

hipError_t launch_linear_bwd(const LinearArgs& a, const Codebook& cb, const uint16_t* dY, const uint16_t* X,
                             const float* XA, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, hipStream_t s) {
  if (a.T == 0) {
    hipError_t e = launch_zero_u16(dA, a.K * a.r, s);
    if (e != hipSuccess) return e;
    return launch_zero_u16(dB, (int64_t)a.r * a.N, s);
  }
  const BwdLayout l = bwd_layout(a.T, a.K, a.N, a.r);
  char* w = reinterpret_cast<char*>(ws);
  float* Pg = reinterpret_cast<float*>(w);
  uint16_t* Gh = reinterpret_cast<uint16_t*>(w + l.pg);
  uint16_t* Gl = reinterpret_cast<uint16_t*>(w + l.pg + l.g);
  char* w2 = w + l.pg + 2 * l.g;
  uint16_t* Gth = reinterpret_cast<uint16_t*>(w2);
  uint16_t* Gtl = reinterpret_cast<uint16_t*>(w2 + l.planes);
  uint16_t* XAth = reinterpret_cast<uint16_t*>(w2 + 2 * l.planes);
  uint16_t* XAtl = reinterpret_cast<uint16_t*>(w2 + 3 * l.planes);
  float* Ptok_b = reinterpret_cast<float*>(w2 + 4 * l.planes);
  float* Ptok_a = reinterpret_cast<float*>(w2 + 4 * l.planes + l.ptok_b);
  char* w3 = w2 + 4 * l.planes + l.ptok_b + l.ptok_a;
  float* slots = reinterpret_cast<float*>(w3);
  int* counters = reinterpret_cast<int*>(w3 + l.slots);
  const SplitPlan dp = dx_plan(a.T, a.K, a.N);
  const int64_t TP = round_up(a.T, 64);

  // G = dY B^T as the bf16 hi / lo rows of s G (the dX GEMM's adapter step)
  // and as transposed hi / lo planes (dA), plus the planes of XA (dB).
  RowdotOut o{};
  o.row_hi = Gh;
  o.row_lo = Gl;
  o.scale_row = a.s;
  o.t_hi = Gth;
  o.t_lo = Gtl;
  o.TP = TP;
  o.side = XA;
  o.side_hi = XAth;
  o.side_lo = XAtl;
  o.zero = counters;  // the dX GEMM's split tickets
  o.nzero = 2 * dp.nsplit();
  hipError_t e = launch_rowdot(dY, a.B, /*v_lr=*/false, Pg, o, a.T, a.N, a.r, row_chunk(a.T, a.N), s);
  if (e != hipSuccess) return e;
  // dB = s XA^T dY (stored [r,N]) and dA = s X^T G (stored [K,r]) in one launch.
  TokJob jb{}, ja{};
  jb.M = dY;
  jb.Sh = XAth;
  jb.Sl = XAtl;
  jb.P = Ptok_b;
  jb.out = dB;
  jb.C = a.N;
  jb.TC = tok_chunk(a.T, a.N);
  jb.scale = a.s;
  jb.m_major = 0;
  ja.M = X;
  ja.Sh = Gth;
  ja.Sl = Gtl;
  ja.P = Ptok_a;
  ja.out = dA;
  ja.C = a.K;
  ja.TC = tok_chunk(a.T, a.K);
  ja.scale = a.s;
  ja.m_major = 1;
  e = launch_tokdot2(jb, ja, a.T, TP, a.r, s);
  if (e != hipSuccess) return e;
  DxGemmParams p{};
  p.status = status_word(&e);
  if (!p.status) return e;
  p.dY = dY;
  p.codes = a.codes;
  p.q8 = a.q8;
  p.s2 = a.s2;
  p.A = a.A;
  p.Gh = Gh;
  p.Gl = Gl;
  p.dX = dX;
  p.T = a.T;
  p.K = a.K;
  p.N = a.N;
  p.r = a.r;
  p.RP = (int)rpad(a.r);
  p.slots = slots;
  p.counters = counters;
  return launch_gemm_dx(p, cb, s);
}

}  // namespace qlora
