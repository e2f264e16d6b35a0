// Serialization of quantized weights (storage.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

enum { kStorageOk = 0, kStorageIo = 1, kStorageMismatch = 2, kStorageHip = 3 };

// Writes codes [N*K/2], q8 [ceil(N*K/64)], s2 [ceil(N*K/64/256)] (device
// pointers) after waiting for `stream`.
int save_4bit(const char* path, int qtype, const float table[16], int64_t N, int64_t K, const uint8_t* codes,
              const uint8_t* q8, const float* s2, hipStream_t stream, hipError_t* herr);

// Reads and validates a file; returns its type and shape.  With codes NULL
// only the header is checked; otherwise the file must hold expect_qtype,
// expect_N, expect_K and the tensors are copied to the device buffers.
int load_4bit(const char* path, const float* const tables[3], int* qtype, int64_t* N, int64_t* K, uint8_t* codes,
              uint8_t* q8, float* s2, int expect_qtype, int64_t expect_N, int64_t expect_K, hipError_t* herr);

}  // namespace qlora
