// Launchers of the LoRA skinny-product kernels (lora.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// Outputs of a rowdot reduction (each optional: null skips it).  RP is r
// rounded up to 64; TP is T rounded up to 64.
struct RowdotOut {
  float* f32;            // [T][r] fp32 result
  uint16_t* row_hi;      // [T][RP] bf16 hi part of scale_row * result
  uint16_t* row_lo;      // [T][RP] bf16 lo part
  float scale_row;
  uint16_t* t_hi;        // [RP][TP] bf16 hi part of the result, transposed
  uint16_t* t_lo;        // [RP][TP] bf16 lo part
  int64_t TP;
  const float* side;     // optional extra [T][r] fp32 input, transposed and split
  uint16_t* side_hi;     // into [RP][TP] hi / lo planes
  uint16_t* side_lo;
  int* zero;             // optional ints set to zero (counters of a later kernel)
  int64_t nzero;
};

// out[T][r] = M[T,L] V  with V = A[L,r] (v_lr) or B[r,L]^T.  P is scratch of
// ceil(L/LC) * T * RP floats; LC a multiple of 128.
hipError_t launch_rowdot(const uint16_t* M, const uint16_t* V, bool v_lr, float* P, const RowdotOut& o, int64_t T,
                         int64_t L, int r, int64_t LC, hipStream_t s);

// out = bf16(scale * M[T,C]^T S[T,r]) stored [r,C] (or [C,r] when m_major),
// with S given as transposed hi / lo planes [RP][TP].  P is scratch of
// ceil(T/TC) * RP * C floats; TC a multiple of 128.
hipError_t launch_tokdot(const uint16_t* M, const uint16_t* Sh, const uint16_t* Sl, int64_t TP, float* P,
                         uint16_t* out, int64_t T, int64_t C, int r, int64_t TC, float scale, bool m_major,
                         hipStream_t s);

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t s);

}  // namespace qlora
