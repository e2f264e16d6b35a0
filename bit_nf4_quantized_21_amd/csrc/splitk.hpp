// Split-contraction combine for the 256 x 256-tile dequant-GEMMs.
//
// A tile's contraction is cut into S slices run by S workgroups.  Every
// slice writes its fp32 accumulators to its own slot of a workspace region,
// then takes a ticket from the tile's counter; the workgroup that draws the
// last ticket sums the S slots in slot order (its own from registers), so the
// result does not depend on which slice finished last, and resets the
// counter to zero for the next launch.  Nothing waits on another workgroup.
#pragma once

#include "common.hpp"

namespace qlora {

constexpr int kSplitSlotFloats = 256 * 256;  // one tile of fp32 partials

// Returns true in the workgroup that must finish the tile (acc then holds the
// full sum); false in the others, which must exit without storing.  Called by
// all NT threads of the workgroup; flag is one int of LDS.
template <int NA, int NB, int NT = 256>
__device__ __forceinline__ bool splitk_combine(f32x16 (&acc)[NA][NB], float* __restrict__ slots, int* counter,
                                               int S, int sidx, int* flag) {
  static_assert(NA * NB * 16 * NT == kSplitSlotFloats, "tile size");
  const int tid = threadIdx.x;
  float4* mine = reinterpret_cast<float4*>(slots) + (int64_t)sidx * (kSplitSlotFloats / 4);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        mine[((a * NB + b) * 4 + e4) * NT + tid] =
            make_float4(acc[a][b][4 * e4], acc[a][b][4 * e4 + 1], acc[a][b][4 * e4 + 2], acc[a][b][4 * e4 + 3]);
  __threadfence();  // this slot is visible device-wide before the ticket
  __syncthreads();
  if (tid == 0) *flag = atomicAdd(counter, 1);
  __syncthreads();
  if (*flag != S - 1) return false;
  __threadfence();  // acquire: the other slots are complete
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t idx = ((a * NB + b) * 4 + e4) * NT + tid;
        const float4 own = make_float4(acc[a][b][4 * e4], acc[a][b][4 * e4 + 1], acc[a][b][4 * e4 + 2],
                                       acc[a][b][4 * e4 + 3]);
        const float4* sl = reinterpret_cast<const float4*>(slots);
        float4 sum = sidx == 0 ? own : sl[idx];
        for (int s = 1; s < S; ++s) {
          const float4 v = s == sidx ? own : sl[(int64_t)s * (kSplitSlotFloats / 4) + idx];
          sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        acc[a][b][4 * e4] = sum.x;
        acc[a][b][4 * e4 + 1] = sum.y;
        acc[a][b][4 * e4 + 2] = sum.z;
        acc[a][b][4 * e4 + 3] = sum.w;
      }
  if (tid == 0) atomicExch(counter, 0);
  return true;
}

// Number of slices for a grid of `tiles` tiles of `steps` contraction steps
// on 256 compute units: split only to fill otherwise idle units (measured on
// the 7B MLP shapes, splitting a grid that already covers the chip costs more
// in partial-sum traffic and per-workgroup start-up than the shorter last
// round saves).
inline int choose_split(int64_t tiles, int64_t steps) {
  int best = 1;
  for (int S = 2; S <= 4; ++S) {
    if (tiles * S > 256 || S > steps) break;
    if ((steps + S - 1) / S * (S - 1) >= steps) continue;  // no empty slice
    best = S;
  }
  return best;
}

}  // namespace qlora
