// Device-resident state of the library: one status word per GPU that kernels
// set when a bounded wait runs out (the host reads and clears it with
// qlora_device_status).
#pragma once

#include <hip/hip_runtime.h>

namespace qlora {

constexpr int kStatusSplitWait = 1;  // a split-contraction finisher stopped waiting for its slices

// Device address of the current device's status word (looked up once per
// device with hipGetSymbolAddress); nullptr with *err set on failure.
int* status_word(hipError_t* err);

// Waits for `s`, returns the current device's status bits and clears them.
hipError_t take_status(hipStream_t s, int* bits);

}  // namespace qlora
