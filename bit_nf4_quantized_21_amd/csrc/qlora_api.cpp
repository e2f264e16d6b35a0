// C ABI of libqlora (declared in include/qlora.h): host-side argument
// validation, the codebook, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qlora.h"
#include "codebook.hpp"
#include "common.hpp"
#include "device_state.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace {

thread_local int g_last_hip_error = 0;

struct Tables {
  qlora::Codebook cb;
  qlora::Midpoints mp;
};

const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] {
    qlora::build_codebook(t.cb.c);
    // Decision boundaries between neighbouring codes, exact in fp64.
    for (int j = 0; j < 15; ++j) t.mp.m[j] = ((double)t.cb.c[j] + (double)t.cb.c[j + 1]) / 2.0;
  });
  return t;
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
  if (out) std::memcpy(out, tables().cb.c, sizeof(float) * 16);
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

int qlora_quantize_nf4(const float* W, int64_t n, int32_t blocksize, uint8_t* codes, float* absmax,
                       void* stream) {
  if (blocksize != 64) return QLORA_ERR_UNSUPPORTED;
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (n == 0) return QLORA_OK;
  if (!W || !codes || !absmax) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_quantize_nf4(W, n, codes, absmax, tables().mp, (hipStream_t)stream));
}

int qlora_quantize_nf4_bf16(const uint16_t* W, int64_t n, int32_t blocksize, uint8_t* codes, float* absmax,
                            void* stream) {
  if (blocksize != 64) return QLORA_ERR_UNSUPPORTED;
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (n == 0) return QLORA_OK;
  if (!W || !codes || !absmax) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_quantize_nf4_bf16(W, n, codes, absmax, tables().mp, (hipStream_t)stream));
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

int qlora_dequantize_nf4(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                         int32_t out_is_bf16, void* out, void* stream) {
  if (n < 0 || n % 2 != 0 || n > (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (out_is_bf16 != 0 && out_is_bf16 != 1) return QLORA_ERR_UNSUPPORTED;
  if (n == 0) return QLORA_OK;
  if (!codes || !q8 || !s2 || !out) return QLORA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(q8) || !aligned16(s2) || !aligned16(out)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_dequantize(codes, q8, s2, n, out_is_bf16, out, tables().cb, (hipStream_t)stream));
}

size_t qlora_linear_fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
  return qlora::fwd_workspace_bytes(T, K, N, r);
}

size_t qlora_linear_bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r) {
  if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
  return qlora::bwd_workspace_bytes(T, K, N, r);
}

int qlora_linear_fwd(const uint16_t* X, int64_t T, int64_t K, int64_t N, const uint8_t* codes, const uint8_t* q8,
                     const float* s2, const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                     float* XA, void* workspace, size_t workspace_bytes, void* stream) {
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
  return hip_status(qlora::launch_linear_fwd(a, tables().cb, X, Y, XA, workspace, (hipStream_t)stream));
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
  return hip_status(qlora::launch_linear_fwd(a, tables().cb, X, Y, XA, ws, (hipStream_t)stream));
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* XA, int64_t T, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* q8, const float* s2, const uint16_t* A, const uint16_t* B,
                     int32_t r, float alpha, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_linear_shape(T, K, N, r);
  if (st != QLORA_OK) return st;
  if (!dA || !dB) return QLORA_ERR_NULL;
  if (T > 0 && (!dY || !X || !XA || !codes || !q8 || !s2 || !A || !B || !dX)) return QLORA_ERR_NULL;
  if (!aligned16(dA) || !aligned16(dB)) return QLORA_ERR_ALIGN;
  if (T > 0 && (!aligned16(dY) || !aligned16(X) || !aligned16(XA) || !aligned16(codes) || !aligned16(q8) ||
                !aligned16(s2) || !aligned16(A) || !aligned16(B) || !aligned16(dX)))
    return QLORA_ERR_ALIGN;
  const size_t need = qlora::bwd_workspace_bytes(T, K, N, r);
  if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  qlora::LinearArgs a{T, K, N, r, (float)(alpha / (float)r), codes, q8, s2, A, B};
  return hip_status(
      qlora::launch_linear_bwd(a, tables().cb, dY, X, XA, dX, dA, dB, workspace, (hipStream_t)stream));
}

}  // extern "C"
