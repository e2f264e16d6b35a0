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

// Scratch of the no-allocation forward entry point: a file-scope device
// array of this many bytes on every GPU the library runs on.
constexpr size_t kNoallocScratchBytes = size_t(80) << 20;

// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress); nullptr with *err set on failure.
void* noalloc_scratch(hipError_t* err);

}  // namespace qlora
