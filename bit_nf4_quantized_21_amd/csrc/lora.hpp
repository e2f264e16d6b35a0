// Launchers of the LoRA skinny-product kernels (lora.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// Outputs of a rowdot reduction (each optional: null skips it).  RP is r
// rounded up to 64; TP is T rounded up to 64.
//
// A "tokdot plane" holds an RP x TP bf16 matrix S^T (element (j, t)) in the
// order the tokdot's MFMAs read it: 16-byte unit
//   u = ((t / 32) * (RP / 16) + j / 16) * 64 + (j % 16) + 16 * ((t % 32) / 8)
// holds t % 8 = 0..7, so one wave's A operand for 32 tokens and 16 rows j is
// 1 KB of consecutive bytes.  Zero outside T x r.
struct RowdotOut {
  float* f32;            // [T][r] fp32 result
  uint16_t* row_hi;      // [T][RP] bf16 hi part of scale_row * result
  uint16_t* row_lo;      // [T][RP] bf16 lo part
  float scale_row;
  uint16_t* t_hi;        // tokdot plane: bf16 hi part of the result
  uint16_t* t_lo;        // tokdot plane: bf16 lo part
  int64_t TP;
  const float* side;     // optional extra [T][r] fp32 input, split into
  uint16_t* side_hi;     // hi / lo tokdot planes
  uint16_t* side_lo;
  int* zero;             // optional ints set to zero (counters of a later kernel)
  int64_t nzero;
};

// Up to kRowdotJobsMax same-shape rowdots in one launch each of the partial
// and the reduction kernels.
constexpr int kRowdotJobsMax = 4;
struct RowdotJobs {
  const uint16_t* M[kRowdotJobsMax];
  const uint16_t* V[kRowdotJobsMax];
  float* P[kRowdotJobsMax];
  int nc;  // chunks of the contraction per job
};
struct RowdotOuts {
  RowdotOut o[kRowdotJobsMax];
};

// out[T][r] = M[T,L] V  with V = A[L,r] (v_lr) or B[r,L]^T.  P is scratch of
// ceil(L/LC) * T * RP floats; LC a multiple of 128.
hipError_t launch_rowdot_batch(int count, const uint16_t* const* M, const uint16_t* const* V, bool v_lr,
                               float* const* P, const RowdotOut* o, int64_t T, int64_t L, int r, int64_t LC,
                               hipStream_t s);
hipError_t launch_rowdot(const uint16_t* M, const uint16_t* V, bool v_lr, float* P, const RowdotOut& o, int64_t T,
                         int64_t L, int r, int64_t LC, hipStream_t s);

// One tokdot: out = bf16(scale * M[T,C]^T S[T,r]) stored [r,C] (or [C,r]
// when m_major), with S given as hi / lo tokdot planes (RowdotOut).  P is
// scratch of ceil(T/TC) * RP * C floats; TC a multiple of 128.  nc and
// mtiles are filled by the launcher.
struct TokJob {
  const uint16_t* M;
  const uint16_t* Sh;
  const uint16_t* Sl;
  float* P;
  uint16_t* out;
  int64_t C, TC;
  float scale;
  int m_major;
  int nc, mtiles;
};

// Up to kTokJobsMax tokdots over the same T tokens and rank r in one launch
// of the partial kernel and one of the reduction (their grids concatenated;
// wg_begin / red_begin are filled by the launcher).
constexpr int kTokJobsMax = 8;
struct TokJobs {
  TokJob j[kTokJobsMax];
  int wg_begin[kTokJobsMax];
  int red_begin[kTokJobsMax];
  int count;
  int r;
};
hipError_t launch_tokdot_n(int count, const TokJob* jobs, int64_t T, int64_t TP, int r, hipStream_t s);
hipError_t launch_tokdot2(const TokJob& a, const TokJob& b, int64_t T, int64_t TP, int r, hipStream_t s);

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t s);

}  // namespace qlora
