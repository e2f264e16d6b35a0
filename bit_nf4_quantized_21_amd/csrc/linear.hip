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

// Workgroups a rank-r launch aims for across all its jobs: one per CU.
constexpr int64_t kRankWGs = 256;

// Chunk of the contraction of a rowdot (X A or dY B^T) of `jobs` same-shape
// problems in one launch: about kRankWGs workgroups of 64 rows each, chunks
// a multiple of 128 long.
int64_t row_chunk(int64_t T, int64_t L, int jobs = 1) {
  const int64_t tiles = cdiv(T, 64) * jobs;
  int64_t nc = cdiv(kRankWGs, tiles);
  const int64_t maxc = cdiv(L, 128);
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  return round_up(cdiv(L, nc), 128);
}

// Token chunk of the tokdots (X^T G, dY^T XA) of one launch, whose jobs
// have `tiles` 64-column tiles in all: about kRankWGs workgroups, chunks a
// multiple of 128 tokens.
int64_t tok_chunk(int64_t T, int64_t tiles) {
  int64_t nc = cdiv(kRankWGs, tiles);
  const int64_t maxc = cdiv(T, 128);
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  return round_up(cdiv(T, nc), 128);
}

// The tokdot chunk of the backward of `count` problems of shape K x N.
int64_t bwd_tok_chunk(int64_t T, int64_t K, int64_t N, int count) {
  return tok_chunk(T, count * (cdiv(K, 64) + cdiv(N, 64)));
}

// Backward workspace regions, each 256-byte aligned.
struct BwdLayout {
  size_t pg, g, planes, ptok_b, ptok_a, slots, counters, xa, pxa, total;
};
// `count` > 1: the per-problem regions of a batch of that many problems.
BwdLayout bwd_layout(int64_t T, int64_t K, int64_t N, int32_t r, int count = 1) {
  BwdLayout l{};
  const int64_t RP = rpad(r), TP = round_up(T, 64);
  l.pg = align256((size_t)cdiv(N, row_chunk(T, N, count)) * T * RP * sizeof(float));
  l.g = align256((size_t)T * RP * sizeof(uint16_t));
  l.planes = align256((size_t)RP * TP * sizeof(uint16_t));
  // a tokdot of one chunk writes its output directly and needs no partials
  const int64_t ntc = cdiv(T, bwd_tok_chunk(T, K, N, count));
  l.ptok_b = ntc > 1 ? align256((size_t)ntc * RP * N * sizeof(float)) : 0;
  l.ptok_a = ntc > 1 ? align256((size_t)ntc * RP * K * sizeof(float)) : 0;
  const SplitPlan dp = dx_plan(T, K, N);
  l.slots = dp.S > 1 ? align256((size_t)dp.nsplit() * dp.S * kSplitSlotFloats * sizeof(float)) : 0;
  l.counters = align256((size_t)(dp.nsplit() > 0 ? 2 * dp.nsplit() : 1) * sizeof(int));
  // recomputation of XA when the caller did not keep it: XA and its rowdot
  // partials
  l.xa = align256((size_t)T * r * sizeof(float));
  l.pxa = align256((size_t)cdiv(K, row_chunk(T, K)) * T * RP * sizeof(float));
  l.total = l.pg + 2 * l.g + 4 * l.planes + l.ptok_b + l.ptok_a + l.slots + l.counters + l.xa + l.pxa;
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

// ---------------------------------------------------------------------------
// Batches of same-shape linears on the GEMM path (T > 16): each linear's
// rank-r products run as usual, then ONE GEMM launch serves all their tiles
// (problem-major tile order, one split plan), so small token counts fill
// the GPU with whole-contraction tiles instead of contraction slices.
// ---------------------------------------------------------------------------
namespace {
static_assert(kGemmBatchMax <= kRowdotJobsMax && 2 * kGemmBatchMax <= kTokJobsMax,
              "a batch's rank-r products fit one launch of each kernel");
struct FwdBatchLayout {
  size_t p, xah, slots, counters, total;
  SplitPlan g;
};
FwdBatchLayout fwd_batch_layout(int64_t T, int64_t K, int64_t N, int32_t r, int count) {
  FwdBatchLayout l{};
  l.p = align256((size_t)cdiv(K, row_chunk(T, K, count)) * T * rpad(r) * sizeof(float));
  l.xah = align256((size_t)T * rpad(r) * sizeof(uint16_t));
  l.g = fwd_plan(T, K, N, count);
  l.slots = l.g.S > 1 ? align256((size_t)l.g.nsplit() * l.g.S * kSplitSlotFloats * sizeof(float)) : 0;
  l.counters = align256((size_t)(l.g.nsplit() > 0 ? 2 * l.g.nsplit() : 1) * sizeof(int));
  // per problem: rowdot partials and the hi / lo rows of s XA
  l.total = (size_t)count * (l.p + 2 * l.xah) + l.slots + l.counters;
  return l;
}
struct BwdBatchLayout {
  size_t pg, g, planes, ptok_b, ptok_a, per, slots, counters, total;
  SplitPlan d;
};
BwdBatchLayout bwd_batch_layout(int64_t T, int64_t K, int64_t N, int32_t r, int count) {
  BwdBatchLayout l{};
  const BwdLayout b = bwd_layout(T, K, N, r, count);
  l.pg = b.pg;
  l.g = b.g;
  l.planes = b.planes;
  l.ptok_b = b.ptok_b;
  l.ptok_a = b.ptok_a;
  l.d = dx_plan(T, K, N, count);
  l.slots = l.d.S > 1 ? align256((size_t)l.d.nsplit() * l.d.S * kSplitSlotFloats * sizeof(float)) : 0;
  l.counters = align256((size_t)(l.d.nsplit() > 0 ? 2 * l.d.nsplit() : 1) * sizeof(int));
  // per problem: rowdot partials, hi / lo rows of s G, four tokdot planes
  // and the two tokdot partial areas
  l.per = l.pg + 2 * l.g + 4 * l.planes + l.ptok_b + l.ptok_a;
  l.total = (size_t)count * l.per + l.slots + l.counters;
  return l;
}
}  // namespace

size_t fwd_batch_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r, int count) {
  if (T <= 0) return 0;
  return fwd_batch_layout(T, K, N, r, count).total;
}
size_t bwd_batch_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r, int count) {
  if (T <= 0) return 0;
  return bwd_batch_layout(T, K, N, r, count).total;
}

hipError_t launch_linear_fwd_batch(int count, const GroupedLinear* L, int64_t T, int32_t r, float s,
                                   const Codebook& cb, void* ws, hipStream_t st) {
  const int64_t K = L[0].K, N = L[0].N;
  const FwdBatchLayout l = fwd_batch_layout(T, K, N, r, count);
  char* w = reinterpret_cast<char*>(ws);
  char* w2 = w + (size_t)count * (l.p + 2 * l.xah);
  int* counters = reinterpret_cast<int*>(w2 + l.slots);
  FwdGemmParams p{};
  hipError_t e = hipSuccess;
  p.status = status_word(&e);
  if (!p.status) return e;
  // XA = X A of every problem: one launch of each rowdot kernel
  const uint16_t* Ms[kRowdotJobsMax];
  const uint16_t* Vs[kRowdotJobsMax];
  float* Ps[kRowdotJobsMax];
  RowdotOut os[kRowdotJobsMax] = {};
  for (int i = 0; i < count; ++i) {
    char* wi = w + (size_t)i * (l.p + 2 * l.xah);
    uint16_t* XAh = reinterpret_cast<uint16_t*>(wi + l.p);
    uint16_t* XAl = reinterpret_cast<uint16_t*>(wi + l.p + l.xah);
    Ms[i] = L[i].X;
    Vs[i] = L[i].A;
    Ps[i] = reinterpret_cast<float*>(wi);
    os[i].f32 = L[i].XA;
    os[i].row_hi = XAh;
    os[i].row_lo = XAl;
    os[i].scale_row = s;
    p.prob[i] = FwdGemmProblem{L[i].X, L[i].codes, L[i].q8, L[i].s2, L[i].B, XAh, XAl, L[i].Y};
  }
  os[0].zero = counters;  // the batched GEMM's split tickets
  os[0].nzero = 2 * l.g.nsplit();
  e = launch_rowdot_batch(count, Ms, Vs, /*v_lr=*/true, Ps, os, T, K, r, row_chunk(T, K, count), st);
  if (e != hipSuccess) return e;
  p.batch = count;
  p.T = T;
  p.K = K;
  p.N = N;
  p.r = r;
  p.s = s;
  p.RP = (int)rpad(r);
  p.slots = reinterpret_cast<float*>(w2);
  p.counters = counters;
  return launch_gemm_fwd_batched(p, cb, st);
}

hipError_t launch_linear_bwd_batch(int count, const GroupedLinearBwd* L, int64_t T, int32_t r, float s,
                                   const Codebook& cb, void* ws, hipStream_t st) {
  const int64_t K = L[0].K, N = L[0].N;
  if (T == 0) {
    for (int i = 0; i < count; ++i) {
      hipError_t e = launch_zero_u16(L[i].dA, K * r, st);
      if (e != hipSuccess) return e;
      e = launch_zero_u16(L[i].dB, (int64_t)r * N, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const BwdBatchLayout l = bwd_batch_layout(T, K, N, r, count);
  char* w = reinterpret_cast<char*>(ws);
  char* w3 = w + (size_t)count * l.per;
  int* counters = reinterpret_cast<int*>(w3 + l.slots);
  const int64_t TP = round_up(T, 64);
  DxGemmParams p{};
  hipError_t e = hipSuccess;
  p.status = status_word(&e);
  if (!p.status) return e;
  const uint16_t* Ms[kRowdotJobsMax];
  const uint16_t* Vs[kRowdotJobsMax];
  float* Ps[kRowdotJobsMax];
  RowdotOut os[kRowdotJobsMax] = {};
  TokJob tj[2 * kRowdotJobsMax] = {};
  for (int i = 0; i < count; ++i) {
    char* wi = w + (size_t)i * l.per;
    uint16_t* Gh = reinterpret_cast<uint16_t*>(wi + l.pg);
    uint16_t* Gl = reinterpret_cast<uint16_t*>(wi + l.pg + l.g);
    char* w2 = wi + l.pg + 2 * l.g;
    uint16_t* Gth = reinterpret_cast<uint16_t*>(w2);
    uint16_t* Gtl = reinterpret_cast<uint16_t*>(w2 + l.planes);
    uint16_t* XAth = reinterpret_cast<uint16_t*>(w2 + 2 * l.planes);
    uint16_t* XAtl = reinterpret_cast<uint16_t*>(w2 + 3 * l.planes);
    Ms[i] = L[i].dY;
    Vs[i] = L[i].B;
    Ps[i] = reinterpret_cast<float*>(wi);
    RowdotOut& o = os[i];
    o.row_hi = Gh;
    o.row_lo = Gl;
    o.scale_row = s;
    o.t_hi = Gth;
    o.t_lo = Gtl;
    o.TP = TP;
    o.side = L[i].XA;
    o.side_hi = XAth;
    o.side_lo = XAtl;
    TokJob& jb = tj[2 * i];
    TokJob& ja = tj[2 * i + 1];
    jb.M = L[i].dY;
    jb.Sh = XAth;
    jb.Sl = XAtl;
    jb.P = reinterpret_cast<float*>(w2 + 4 * l.planes);
    jb.out = L[i].dB;
    jb.C = N;
    jb.TC = bwd_tok_chunk(T, K, N, count);
    jb.scale = s;
    jb.m_major = 0;
    ja.M = L[i].X;
    ja.Sh = Gth;
    ja.Sl = Gtl;
    ja.P = reinterpret_cast<float*>(w2 + 4 * l.planes + l.ptok_b);
    ja.out = L[i].dA;
    ja.C = K;
    ja.TC = bwd_tok_chunk(T, K, N, count);
    ja.scale = s;
    ja.m_major = 1;
    p.prob[i] = DxGemmProblem{L[i].dY, L[i].codes, L[i].q8, L[i].s2, L[i].A, Gh, Gl, L[i].dX};
  }
  os[0].zero = counters;  // the batched dX GEMM's split tickets
  os[0].nzero = 2 * l.d.nsplit();
  // G = dY B^T of every problem, then dB and dA of every problem: one launch
  // of each kernel
  e = launch_rowdot_batch(count, Ms, Vs, /*v_lr=*/false, Ps, os, T, N, r, row_chunk(T, N, count), st);
  if (e != hipSuccess) return e;
  e = launch_tokdot_n(2 * count, tj, T, TP, r, st);
  if (e != hipSuccess) return e;
  p.batch = count;
  p.T = T;
  p.K = K;
  p.N = N;
  p.r = r;
  p.RP = (int)rpad(r);
  p.slots = reinterpret_cast<float*>(w3);
  p.counters = counters;
  return launch_gemm_dx_batched(p, cb, st);
}

// Runs of consecutive linears with the same K and N, at most kGemmBatchMax
// long, in order; calls f(first, count) for each.
template <class L, class F>
static hipError_t for_each_run(int count, const L* x, F f) {
  for (int i = 0; i < count;) {
    int n = 1;
    while (i + n < count && n < kGemmBatchMax && x[i + n].K == x[i].K && x[i + n].N == x[i].N) ++n;
    hipError_t e = f(i, n);
    if (e != hipSuccess) return e;
    i += n;
  }
  return hipSuccess;
}

size_t bwd_grouped_workspace_bytes(int count, const GroupedLinearBwd* L, int64_t T, int32_t r) {
  size_t total = 0;
  for_each_run(count, L, [&](int i, int n) {
    const size_t b = bwd_batch_workspace_bytes(T, L[i].K, L[i].N, r, n);
    total = total > b ? total : b;
    return hipSuccess;
  });
  return total;
}

hipError_t launch_linear_bwd_grouped(int count, const GroupedLinearBwd* L, int64_t T, int32_t r, float s,
                                     const Codebook& cb, void* ws, hipStream_t st) {
  return for_each_run(count, L, [&](int i, int n) { return launch_linear_bwd_batch(n, L + i, T, r, s, cb, ws, st); });
}

// Grouped small-token forward: T <= 16 runs every chunk of up to
// kGemvGroupMax linears as one XA-partial launch and one GEMV launch, each
// linear's partials in its own workspace region; larger T runs each linear's
// GEMM path in turn on the shared workspace.
size_t fwd_grouped_workspace_bytes(int count, const GroupedLinear* L, int64_t T, int32_t r) {
  if (T <= 0) return 0;
  size_t total = 0;
  if (T <= kGemvMaxT) {
    for (int i = 0; i < count; ++i) total += fwd_layout(T, L[i].K, L[i].N, r).total;
    return total;
  }
  for_each_run(count, L, [&](int i, int n) {
    const size_t b = fwd_batch_workspace_bytes(T, L[i].K, L[i].N, r, n);
    total = total > b ? total : b;
    return hipSuccess;
  });
  return total;
}

hipError_t launch_linear_fwd_grouped(int count, const GroupedLinear* L, int64_t T, int32_t r, float s,
                                     const Codebook& cb, void* ws, hipStream_t st) {
  if (T == 0 || count == 0) return hipSuccess;
  char* w = reinterpret_cast<char*>(ws);
  if (T > kGemvMaxT)
    return for_each_run(count, L, [&](int i, int n) { return launch_linear_fwd_batch(n, L + i, T, r, s, cb, ws, st); });
  for (int i0 = 0; i0 < count; i0 += kGemvGroupMax) {
    GemvGroup g{};
    g.count = count - i0 < kGemvGroupMax ? count - i0 : kGemvGroupMax;
    g.T = (int)T;
    g.r = r;
    g.RP = (int)rpad(r);
    g.s = s;
    for (int j = 0; j < g.count; ++j) {
      const GroupedLinear& x = L[i0 + j];
      GemvLinear& y = g.L[j];
      y.X = x.X;
      y.codes = x.codes;
      y.q8 = x.q8;
      y.s2 = x.s2;
      y.A = x.A;
      y.B = x.B;
      y.Y = x.Y;
      y.XA = x.XA;
      y.K = x.K;
      y.N = x.N;
      y.P = reinterpret_cast<float*>(w);
      w += fwd_layout(T, x.K, x.N, r).total;
    }
    hipError_t e = launch_gemv_group(g, cb, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  if (!XA) {
    // Gradient checkpointing: the forward's XA was not kept, so recompute
    // it from X and A (the same kernels and order as the forward, so the
    // value is the forward's bit for bit).
    float* xa = reinterpret_cast<float*>(w3 + l.slots + l.counters);
    RowdotOut ox{};
    ox.f32 = xa;
    hipError_t e0 = launch_rowdot(X, a.A, /*v_lr=*/true, reinterpret_cast<float*>(w3 + l.slots + l.counters + l.xa),
                                  ox, a.T, a.K, a.r, row_chunk(a.T, a.K), s);
    if (e0 != hipSuccess) return e0;
    XA = xa;
  }

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
  jb.TC = bwd_tok_chunk(a.T, a.K, a.N, 1);
  jb.scale = a.s;
  jb.m_major = 0;
  ja.M = X;
  ja.Sh = Gth;
  ja.Sl = Gtl;
  ja.P = Ptok_a;
  ja.out = dA;
  ja.C = a.K;
  ja.TC = bwd_tok_chunk(a.T, a.K, a.N, 1);
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
