// Device-resident state of the library (see device_state.hpp).
//
// The status word is a file-scope __device__ variable: every GPU that loads
// the library holds its own copy at its own address.  In host code the
// variable's name is only a stand-in for that address, so host code never
// passes it to a kernel or a copy; it looks the address up once per device
// with hipGetSymbolAddress and uses that pointer.
#include "device_state.hpp"

#include <mutex>

namespace qlora {

namespace {
__device__ __align__(256) int g_status_word;

// Workspace of qlora_linear_fwd_noalloc, for callers that cannot allocate
// device memory (graph capture, tight serving loops).  Every GPU holds its
// own copy until the process ends; every call on a GPU shares it.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int* g_status_ptr[kMaxDevices] = {};
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int* status_word(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_status_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_status_word));
    if (e != hipSuccess) {
      *err = e;
      return nullptr;
    }
    g_status_ptr[dev] = static_cast<int*>(p);
  }
  *err = hipSuccess;
  return g_status_ptr[dev];
}

void* noalloc_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

hipError_t take_status(hipStream_t s, int* bits) {
  hipError_t e = hipSuccess;
  int* p = status_word(&e);
  if (!p) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpy(&v, p, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  if (v != 0) {
    const int zero = 0;
    e = hipMemcpy(p, &zero, sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
  }
  *bits = v;
  return hipSuccess;
}

}  // namespace qlora
