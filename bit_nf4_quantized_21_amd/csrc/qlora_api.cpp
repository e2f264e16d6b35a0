// C ABI of libqlora (declared in include/qlora.h): host-side argument
// validation, the codebook, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlora.h"
#include "codebook.hpp"
#include "common.hpp"
#include "device_state.hpp"
#include "kernels.hpp"
#include "storage.hpp"
#include "timing.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// Decode table and decision data of each stored 4-bit type, built once.
struct TypeTables {
  qlora::Codebook cb;
  qlora::Midpoints mp;
  bool exact;  // every level boundary times a 24-bit absmax is exact in fp64
};

// Significant bits of a finite double (0 for 0).
int significant_bits(double x) {
  if (x == 0.0) return 0;
  int e = 0;
  double f = std::frexp(std::fabs(x), &e);  // f in [0.5, 1)
  int bits = 0;
  while (f != 0.0 && bits < 64) {
    f = f * 2.0;
    const double d = std::floor(f);
    f -= d;
    ++bits;
  }
  return bits;
}

struct Tables {
  TypeTables t[qlora::kQTypes];
};

const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] {
    for (int q = 0; q < qlora::kQTypes; ++q) {
      TypeTables& tt = t.t[q];
      qlora::build_type_table(q, tt.cb.c);
      qlora::TypeLevels lv{};
      qlora::build_type_levels(q, tt.cb.c, &lv);
      tt.exact = true;
      tt.mp.codes = 0;
      for (int i = 0; i < lv.n; ++i) tt.mp.codes |= (uint64_t)lv.code[i] << (4 * i);
      for (int i = lv.n; i < 16; ++i) tt.mp.codes |= (uint64_t)lv.code[lv.n - 1] << (4 * i);
      tt.mp.zero_code = lv.zero_code;
      // Boundaries between neighbouring levels, exact in fp64 (two fp32
      // values a few binades apart add exactly; halving is exact).
      for (int j = 0; j < 15; ++j) {
        if (j + 1 < lv.n) {
          tt.mp.m[j] = ((double)lv.level[j] + (double)lv.level[j + 1]) / 2.0;
          if (significant_bits(tt.mp.m[j]) > 29) tt.exact = false;
        } else {
          tt.mp.m[j] = HUGE_VAL;
        }
      }
    }
  });
  return t;
}

const TypeTables* type_tables(int32_t qtype) {
  if (qtype < 0 || qtype >= qlora::kQTypes) return nullptr;
  const TypeTables& tt = tables().t[qtype];
  return tt.exact ? &tt : nullptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QLORA_OK;
  g_last_hip_error = (int)e;
  return QLORA_ERR_HIP;
}

int check_linear_shape(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (T < 0 || K < 64 || N < 8) return QLORA_ERR_SHAPE;
  if (K % 64 != 0 || N % 8 != 0) return QLORA_ERR_SHAPE;
  if (T > (int64_t(1) << 31) || K > (int64_t(1) << 28) || N > (int64_t(1) << 28)) return QLORA_ERR_SHAPE;
  if (r < 8 || r > 128 || r % 8 != 0) return QLORA_ERR_UNSUPPORTED;
  if (!qlora::linear_views_fit(T, K, N, r)) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

}  // namespace

extern "C" {

void qlora_nf4_codebook(float out[16]) {
  if (out) std::memcpy(out, tables().t[qlora::kQNF4].cb.c, sizeof(float) * 16);
}

int qlora_4bit_table(int32_t qtype, float out[16]) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (!out) return QLORA_ERR_NULL;
  std::memcpy(out, tt->cb.c, sizeof(float) * 16);
  return QLORA_OK;
}

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_NULL: return "QLORA_ERR_NULL: a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "QLORA_ERR_SHAPE: invalid size (negative, zero or not a required multiple)";
    case QLORA_ERR_ALIGN: return "QLORA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case QLORA_ERR_UNSUPPORTED: return "QLORA_ERR_UNSUPPORTED: unsupported blocksize or rank";
    case QLORA_ERR_HIP: return "QLORA_ERR_HIP: a HIP call failed (see qlora_last_hip_error)";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace missing or too small";
    case QLORA_ERR_IO: return "QLORA_ERR_IO: file missing, unreadable, malformed or of another shape or type";
    case QLORA_ERR_SCRATCH:
      return "QLORA_ERR_SCRATCH: the problem needs more scratch than the no-allocation entry point holds";
    case QLORA_ERR_DEVICE:
      return "QLORA_ERR_DEVICE: a kernel's bounded wait ran out; results since the last status query are unreliable";
    default: return "unknown qlora_status";
  }
}

int qlora_last_hip_error(void) { return g_last_hip_error; }

int qlora_device_status(void* stream) {
  int bits = 0;
  const int st = hip_status(qlora::take_status((hipStream_t)stream, &bits));
  if (st != QLORA_OK) return st;
  return bits ? QLORA_ERR_DEVICE : QLORA_OK;
}

void qlora_timing_enable(int on) { qlora::timing_enable(on != 0); }

int qlora_timing_read(char* buf, size_t buflen) {
  hipError_t e = hipSuccess;
  const std::string text = qlora::timing_collect(&e);
  if (buf && buflen) {
    const size_t n = text.size() < buflen - 1 ? text.size() : buflen - 1;
    std::memcpy(buf, text.data(), n);
    buf[n] = '\0';
  }
  if (e != hipSuccess) return hip_status(e);
  return (int)text.size();
}

int qlora_quantize_4bit(const void* W, int32_t w_is_bf16, int64_t n, int32_t blocksize, int32_t qtype,
                        uint8_t* codes, float* absmax, void* stream) {
  if (blocksize != 64 || (w_is_bf16 != 0 && w_is_bf16 != 1)) return QLORA_ERR_UNSUPPORTED;
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (n == 0) return QLORA_OK;
  if (!W || !codes || !absmax) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  if (w_is_bf16)
    return hip_status(qlora::launch_quantize_nf4_bf16(static_cast<const uint16_t*>(W), n, codes, absmax, tt->mp,
                                                      (hipStream_t)stream));
  return hip_status(
      qlora::launch_quantize_nf4(static_cast<const float*>(W), n, codes, absmax, tt->mp, (hipStream_t)stream));
}

int qlora_quantize_nf4(const float* W, int64_t n, int32_t blocksize, uint8_t* codes, float* absmax,
                       void* stream) {
  return qlora_quantize_4bit(W, 0, n, blocksize, qlora::kQNF4, codes, absmax, stream);
}

int qlora_quantize_nf4_bf16(const uint16_t* W, int64_t n, int32_t blocksize, uint8_t* codes, float* absmax,
                            void* stream) {
  return qlora_quantize_4bit(W, 1, n, blocksize, qlora::kQNF4, codes, absmax, stream);
}

int qlora_quantize_dq(const void* W, int32_t w_is_bf16, int64_t n, int32_t qtype, uint8_t* codes, uint8_t* q8,
                      float* s2, void* stream) {
  if (w_is_bf16 != 0 && w_is_bf16 != 1) return QLORA_ERR_UNSUPPORTED;
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (n == 0) return QLORA_OK;
  if (!W || !codes || !q8 || !s2) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(q8) || !aligned16(s2)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_quantize_dq(W, w_is_bf16 != 0, n, codes, q8, s2, tt->mp, (hipStream_t)stream));
}

int qlora_double_quant(const float* absmax, int64_t nb, int32_t blocksize2, uint8_t* q8, float* s2,
                       void* stream) {
  if (blocksize2 != 256) return QLORA_ERR_UNSUPPORTED;
  if (nb < 0 || nb > (int64_t(1) << 38)) return QLORA_ERR_SHAPE;
  if (nb == 0) return QLORA_OK;
  if (!absmax || !q8 || !s2) return QLORA_ERR_NULL;
  if (!aligned16(absmax) || !aligned16(q8) || !aligned16(s2)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_double_quant(absmax, nb, q8, s2, (hipStream_t)stream));
}

int qlora_dequantize_4bit(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n, int32_t qtype,
                          int32_t out_is_bf16, void* out, void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (out_is_bf16 != 0 && out_is_bf16 != 1) return QLORA_ERR_UNSUPPORTED;
  if (n == 0) return QLORA_OK;
  if (!codes || !q8 || !s2 || !out) return QLORA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(q8) || !aligned16(s2) || !aligned16(out)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_dequantize(codes, q8, s2, n, out_is_bf16, out, tt->cb, (hipStream_t)stream));
}

int qlora_dequantize_nf4(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                         int32_t out_is_bf16, void* out, void* stream) {
  return qlora_dequantize_4bit(codes, q8, s2, n, qlora::kQNF4, out_is_bf16, out, stream);
}

size_t qlora_linear_fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
  return qlora::fwd_workspace_bytes(T, K, N, r);
}

size_t qlora_linear_bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
  return qlora::bwd_workspace_bytes(T, K, N, r);
}

int qlora_linear_fwd_4bit(int32_t qtype, const uint16_t* X, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                          const uint8_t* q8, const float* s2, const uint16_t* A, const uint16_t* B, int32_t r,
                          float alpha, uint16_t* Y, float* XA, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  int st = check_linear_shape(T, K, N, r);
  if (st != QLORA_OK) return st;
  if (T == 0) return QLORA_OK;
  if (!X || !codes || !q8 || !s2 || !A || !B || !Y || !XA) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(q8) || !aligned16(s2) || !aligned16(A) || !aligned16(B) ||
      !aligned16(Y) || !aligned16(XA))
    return QLORA_ERR_ALIGN;
  const size_t need = qlora::fwd_workspace_bytes(T, K, N, r);
  if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  qlora::LinearArgs a{T, K, N, r, (float)(alpha / (float)r), codes, q8, s2, A, B};
  return hip_status(qlora::launch_linear_fwd(a, tt->cb, X, Y, XA, workspace, (hipStream_t)stream));
}

int qlora_linear_fwd(const uint16_t* X, int64_t T, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* q8,
                     const float* s2, const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                     float* XA, void* workspace, size_t workspace_bytes, void* stream) {
  return qlora_linear_fwd_4bit(qlora::kQNF4, X, T, K, N, codes, q8, s2, A, B, r, alpha, Y, XA, workspace,
                               workspace_bytes, stream);
}

namespace {
// Validates a group and converts it; returns a qlora_status.
int check_group(int32_t count, const qlora_linear_desc* d, int64_t T, int32_t r,
                std::vector<qlora::GroupedLinear>* out) {
  if (count < 0 || count > 4096) return QLORA_ERR_SHAPE;
  if (count > 0 && !d) return QLORA_ERR_NULL;
  out->resize((size_t)count);
  for (int i = 0; i < count; ++i) {
    const qlora_linear_desc& x = d[i];
    int st = check_linear_shape(T, x.K, x.N, r);
    if (st != QLORA_OK) return st;
    if (T > 0) {
      if (!x.X || !x.codes || !x.q8 || !x.s2 || !x.A || !x.B || !x.Y || !x.XA) return QLORA_ERR_NULL;
      if (!aligned16(x.X) || !aligned16(x.codes) || !aligned16(x.q8) || !aligned16(x.s2) || !aligned16(x.A) ||
          !aligned16(x.B) || !aligned16(x.Y) || !aligned16(x.XA))
        return QLORA_ERR_ALIGN;
    }
    (*out)[i] = qlora::GroupedLinear{x.X, x.codes, x.q8, x.s2, x.A, x.B, x.Y, x.XA, x.K, x.N};
  }
  return QLORA_OK;
}
}  // namespace

size_t qlora_linear_fwd_grouped_workspace_bytes(int32_t count, const qlora_linear_desc* descs, int64_t T,
                                                 int32_t r) {
  // Only the shapes matter for the size; the pointers are not looked at.
  if (count < 0 || count > 4096 || (count > 0 && !descs) || T < 0) return 0;
  std::vector<qlora::GroupedLinear> g((size_t)count);
  for (int i = 0; i < count; ++i) {
    if (check_linear_shape(T, descs[i].K, descs[i].N, r) != QLORA_OK) return 0;
    g[i].K = descs[i].K;
    g[i].N = descs[i].N;
  }
  return qlora::fwd_grouped_workspace_bytes(count, g.data(), T, r);
}

int qlora_linear_fwd_grouped(int32_t qtype, int32_t count, const qlora_linear_desc* descs, int64_t T, int32_t r,
                             float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (T < 0) return QLORA_ERR_SHAPE;
  std::vector<qlora::GroupedLinear> g;
  int st = check_group(count, descs, T, r, &g);
  if (st != QLORA_OK) return st;
  if (T == 0 || count == 0) return QLORA_OK;
  const size_t need = qlora::fwd_grouped_workspace_bytes(count, g.data(), T, r);
  if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_linear_fwd_grouped(count, g.data(), T, r, (float)(alpha / (float)r), tt->cb,
                                                     workspace, (hipStream_t)stream));
}

namespace {
int check_group_bwd(int32_t count, const qlora_linear_bwd_desc* d, int64_t T, int32_t r,
                    std::vector<qlora::GroupedLinearBwd>* out) {
  if (count < 0 || count > 4096) return QLORA_ERR_SHAPE;
  if (count > 0 && !d) return QLORA_ERR_NULL;
  out->resize((size_t)count);
  for (int i = 0; i < count; ++i) {
    const qlora_linear_bwd_desc& x = d[i];
    int st = check_linear_shape(T, x.K, x.N, r);
    if (st != QLORA_OK) return st;
    if (!x.dA || !x.dB) return QLORA_ERR_NULL;
    if (!aligned16(x.dA) || !aligned16(x.dB)) return QLORA_ERR_ALIGN;
    if (T > 0) {
      if (!x.dY || !x.X || !x.XA || !x.codes || !x.q8 || !x.s2 || !x.A || !x.B || !x.dX) return QLORA_ERR_NULL;
      if (!aligned16(x.dY) || !aligned16(x.X) || !aligned16(x.XA) || !aligned16(x.codes) || !aligned16(x.q8) ||
          !aligned16(x.s2) || !aligned16(x.A) || !aligned16(x.B) || !aligned16(x.dX))
        return QLORA_ERR_ALIGN;
    }
    (*out)[i] = qlora::GroupedLinearBwd{x.dY, x.X, x.XA, x.codes, x.q8, x.s2, x.A, x.B, x.dX, x.dA, x.dB, x.K, x.N};
  }
  return QLORA_OK;
}
}  // namespace

size_t qlora_linear_bwd_grouped_workspace_bytes(int32_t count, const qlora_linear_bwd_desc* descs, int64_t T,
                                                 int32_t r) {
  if (count < 0 || count > 4096 || (count > 0 && !descs) || T < 0) return 0;
  std::vector<qlora::GroupedLinearBwd> g((size_t)count);
  for (int i = 0; i < count; ++i) {
    if (check_linear_shape(T, descs[i].K, descs[i].N, r) != QLORA_OK) return 0;
    g[i].K = descs[i].K;
    g[i].N = descs[i].N;
  }
  if (T == 0) return 0;
  return qlora::bwd_grouped_workspace_bytes(count, g.data(), T, r);
}

int qlora_linear_bwd_grouped(int32_t qtype, int32_t count, const qlora_linear_bwd_desc* descs, int64_t T, int32_t r,
                             float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (T < 0) return QLORA_ERR_SHAPE;
  std::vector<qlora::GroupedLinearBwd> g;
  int st = check_group_bwd(count, descs, T, r, &g);
  if (st != QLORA_OK) return st;
  if (count == 0) return QLORA_OK;
  const size_t need = T > 0 ? qlora::bwd_grouped_workspace_bytes(count, g.data(), T, r) : 0;
  if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_linear_bwd_grouped(count, g.data(), T, r, (float)(alpha / (float)r), tt->cb,
                                                     workspace, (hipStream_t)stream));
}

namespace {
// The device address of a buffer given as device memory or as pinned host
// memory mapped into the device's address space; nullptr if it is neither.
void* device_view(void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice) return p;
  if (at.type == hipMemoryTypeHost) {
    if (at.devicePointer) return at.devicePointer;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}
}  // namespace

size_t qlora_adamw_workspace_bytes(int64_t n) { return n > 0 ? qlora::adamw_workspace_bytes(n) : 0; }

int qlora_adamw_step(int64_t n, uint16_t* param, float* master, float* m, float* v, const uint16_t* grad,
                     int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                     float max_grad_norm, float* grad_norm_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (n < 0 || step < 1) return QLORA_ERR_SHAPE;
  if (!(lr >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
      !(weight_decay >= 0.0f) || !std::isfinite(lr) || !std::isfinite(max_grad_norm))
    return QLORA_ERR_UNSUPPORTED;
  if (n == 0) return QLORA_OK;
  if (!param || !master || !m || !v || !grad) return QLORA_ERR_NULL;
  if (!aligned16(param) || !aligned16(master) || !aligned16(m) || !aligned16(v) || !aligned16(grad) ||
      (grad_norm_out && (reinterpret_cast<uintptr_t>(grad_norm_out) & 3u)))
    return QLORA_ERR_ALIGN;
  const bool need_ws = max_grad_norm > 0.0f || grad_norm_out;
  if (need_ws && (!workspace || workspace_bytes < qlora::adamw_workspace_bytes(n))) return QLORA_ERR_WORKSPACE;
  if (need_ws && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  // Optimizer state may be paged out to pinned host memory.
  float* dm = static_cast<float*>(device_view(master));
  float* d1 = static_cast<float*>(device_view(m));
  float* d2 = static_cast<float*>(device_view(v));
  if (!dm || !d1 || !d2) return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_adamw(n, param, dm, d1, d2, grad, step, lr, beta1, beta2, eps, weight_decay,
                                        max_grad_norm, grad_norm_out, workspace, (hipStream_t)stream));
}

int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                             const uint8_t* q8, const float* s2, const uint16_t* A, const uint16_t* B, int32_t r,
                             float alpha, uint16_t* Y, float* XA, void* stream) {
  int st = check_linear_shape(T, K, N, r);
  if (st != QLORA_OK) return st;
  if (T == 0) return QLORA_OK;
  if (!X || !codes || !q8 || !s2 || !A || !B || !Y || !XA) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(q8) || !aligned16(s2) || !aligned16(A) || !aligned16(B) ||
      !aligned16(Y) || !aligned16(XA))
    return QLORA_ERR_ALIGN;
  if (qlora::fwd_workspace_bytes(T, K, N, r) > qlora::kNoallocScratchBytes) return QLORA_ERR_SCRATCH;
  hipError_t e = hipSuccess;
  void* ws = qlora::noalloc_scratch(&e);
  if (!ws) return hip_status(e);
  qlora::LinearArgs a{T, K, N, r, (float)(alpha / (float)r), codes, q8, s2, A, B};
  return hip_status(qlora::launch_linear_fwd(a, tables().t[qlora::kQNF4].cb, X, Y, XA, ws, (hipStream_t)stream));
}

int qlora_linear_bwd_4bit(int32_t qtype, const uint16_t* dY, const uint16_t* X, const float* XA, int64_t T,
                          int64_t K, int64_t N, const uint8_t* codes, const uint8_t* q8, const float* s2,
                          const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* dX, uint16_t* dA,
                          uint16_t* dB, void* workspace, size_t workspace_bytes, void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  int st = check_linear_shape(T, K, N, r);
  if (st != QLORA_OK) return st;
  if (!dA || !dB) return QLORA_ERR_NULL;
  if (T > 0 && (!dY || !X || !codes || !q8 || !s2 || !A || !B || !dX)) return QLORA_ERR_NULL;  // XA may be NULL
  if (!aligned16(dA) || !aligned16(dB)) return QLORA_ERR_ALIGN;
  if (T > 0 && (!aligned16(dY) || !aligned16(X) || !aligned16(XA) || !aligned16(codes) || !aligned16(q8) ||
                !aligned16(s2) || !aligned16(A) || !aligned16(B) || !aligned16(dX)))
    return QLORA_ERR_ALIGN;
  const size_t need = qlora::bwd_workspace_bytes(T, K, N, r);
  if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  qlora::LinearArgs a{T, K, N, r, (float)(alpha / (float)r), codes, q8, s2, A, B};
  return hip_status(qlora::launch_linear_bwd(a, tt->cb, dY, X, XA, dX, dA, dB, workspace, (hipStream_t)stream));
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* XA, int64_t T, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* q8, const float* s2, const uint16_t* A, const uint16_t* B,
                     int32_t r, float alpha, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return qlora_linear_bwd_4bit(qlora::kQNF4, dY, X, XA, T, K, N, codes, q8, s2, A, B, r, alpha, dX, dA, dB, workspace,
                               workspace_bytes, stream);
}

int qlora_save_4bit(const char* path, int32_t qtype, int64_t N, int64_t K, const uint8_t* codes, const uint8_t* q8,
                    const float* s2, void* stream) {
  const TypeTables* tt = type_tables(qtype);
  if (!tt) return QLORA_ERR_UNSUPPORTED;
  if (N <= 0 || K <= 0 || (N * K) % 2 != 0 || N > (int64_t(1) << 28) || K > (int64_t(1) << 28)) return QLORA_ERR_SHAPE;
  if (!path || !codes || !q8 || !s2) return QLORA_ERR_NULL;
  hipError_t e = hipSuccess;
  const int rc = qlora::save_4bit(path, qtype, tt->cb.c, N, K, codes, q8, s2, (hipStream_t)stream, &e);
  if (rc == qlora::kStorageHip) return hip_status(e);
  return rc == qlora::kStorageOk ? QLORA_OK : QLORA_ERR_IO;
}

int qlora_load_4bit_info(const char* path, int32_t* qtype, int64_t* N, int64_t* K) {
  if (!path || !qtype || !N || !K) return QLORA_ERR_NULL;
  const float* tabs[3] = {tables().t[0].cb.c, tables().t[1].cb.c, tables().t[2].cb.c};
  int q = 0;
  hipError_t e = hipSuccess;
  const int rc = qlora::load_4bit(path, tabs, &q, N, K, nullptr, nullptr, nullptr, 0, 0, 0, &e);
  if (rc != qlora::kStorageOk) return QLORA_ERR_IO;
  *qtype = q;
  return QLORA_OK;
}

int qlora_load_4bit(const char* path, int32_t qtype, int64_t N, int64_t K, uint8_t* codes, uint8_t* q8, float* s2,
                    void* stream) {
  if (!type_tables(qtype)) return QLORA_ERR_UNSUPPORTED;
  if (!path || !codes || !q8 || !s2) return QLORA_ERR_NULL;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  const float* tabs[3] = {tables().t[0].cb.c, tables().t[1].cb.c, tables().t[2].cb.c};
  int q = 0;
  int64_t n_ = 0, k_ = 0;
  const int rc = qlora::load_4bit(path, tabs, &q, &n_, &k_, codes, q8, s2, qtype, N, K, &e);
  if (rc == qlora::kStorageHip) return hip_status(e);
  return rc == qlora::kStorageOk ? QLORA_OK : QLORA_ERR_IO;
}

}  // extern "C"
