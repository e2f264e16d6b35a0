// Launchers of the LoRA skinny-GEMM kernels (lora.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// out[T,r] (fp32) = M[T,L] * V  with V = A[L,r] (v_kmajor) or B[r,L]^T;
// P is scratch of ceil(L/LC)*T*r floats; LC a multiple of 32.
hipError_t launch_rowdot(const uint16_t* M, const uint16_t* V, bool v_kmajor, float* P, float* out, int64_t T,
                         int64_t L, int r, int64_t LC, hipStream_t s);

// out = bf16(scale * M[T,C]^T S[T,r]) stored [C,r] (or [r,C] when transpose);
// P is scratch of ceil(T/TC)*C*r floats; TC a multiple of 32.
hipError_t launch_tokdot(const uint16_t* M, const float* S, float* P, uint16_t* out, int64_t T, int64_t C, int r,
                         int64_t TC, float scale, bool transpose, hipStream_t s);

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t s);

}  // namespace qlora
