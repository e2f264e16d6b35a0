// Optional per-kernel timing with HIP events recorded on the launch stream.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

namespace qlora {

bool timing_enabled();
void timing_enable(bool on);
// Formats "name count total_ms" lines for every kernel timed since the last
// call, after waiting for their events; then forgets them.
std::string timing_collect(hipError_t* err);

// RAII bracket around one kernel launch.  No-op when timing is disabled.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int slot_ = -1;
  hipStream_t s_;
};

}  // namespace qlora
