// Split-contraction combine for the 256 x 256-tile dequant-GEMMs.
//
// A tile's contraction is cut into S slices run by S workgroups.  A slice
// that has finished its part draws a ticket from the tile's counter; all but
// the last ticket write their fp32 accumulators to their own slot of a
// workspace region and then bump the tile's published count.  The last
// ticket waits until the other S - 1 slices have published (they drew their
// tickets first, so they are running and need nothing from anyone to finish),
// sums the S parts in slot order (its own from registers), so the result does
// not depend on which slice finished last, and resets both counts to zero
// for the next launch.  Only S - 1 slices write partials.
//
// Slots and counts are accessed with system-scope cache policy (stores and
// loads that no XCD's caches keep, atomics at the coherence point), so the
// hand-off holds wherever the slices run and no cache has to be written back
// or invalidated: a device-scope fence would write back and invalidate the
// whole L2 of the XCD, which stalls every workgroup on it.
#pragma once

#include "common.hpp"
#include "device_state.hpp"

namespace qlora {

constexpr int kSplitSlotFloats = 256 * 256;  // one tile of fp32 partials
constexpr int kCachePolicySystem = 1 | 16;   // sc0 | sc1

// Adds the partials of the other S - 1 slots (NO >= S - 1 of them) to acc,
// summing every element in slot order with this slot's own value at
// position sidx.  The 16-byte chunks are read KB at a time with the loads of
// all slots of a batch in flight together: one memory round trip per batch,
// not per chunk.
template <int NO, int KB, int NA, int NB, int NT = 256>
__device__ __forceinline__ void splitk_add_slots(f32x16 (&acc)[NA][NB], rsrc_t rs, int S, int sidx) {
  constexpr int kChunks = NA * NB * 4;
  static_assert(kChunks % KB == 0, "batch");
  const int tid = threadIdx.x;
#pragma unroll
  for (int c0 = 0; c0 < kChunks; c0 += KB) {
    u32x4 v[NO][KB];
#pragma unroll
    for (int k = 0; k < NO; ++k) {
      const int s = k < sidx ? k : k + 1;  // k-th slot other than sidx
      if (s < S) {
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const uint32_t off = (uint32_t)(s * kSplitSlotFloats * 4 + ((c0 + i) * NT + tid) * 16);
          v[k][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0,
                                                                                     kCachePolicySystem));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int c = c0 + i, a = c / (NB * 4), b = (c / 4) % NB, e4 = c % 4;
      float sum[4];
#pragma unroll
      for (int s = 0; s <= NO; ++s) {
        if (s >= S) break;  // uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float other = __uint_as_float(s < sidx ? v[s < NO ? s : NO - 1][i][e] : v[s > 0 ? s - 1 : 0][i][e]);
          const float x = s == sidx ? acc[a][b][4 * e4 + e] : other;
          sum[e] = s == 0 ? x : sum[e] + x;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[a][b][4 * e4 + e] = sum[e];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batches apart (registers)
  }
}

// Returns true in the workgroup that must finish the tile (acc then holds the
// full sum); false in the others, which must exit without storing.  Called by
// all NT threads of the workgroup; flag is one int of LDS.  `ticket` and
// `published` are the tile's two counts (zero on entry, left zero).
// `status` is the device's status word: if the finisher's bounded wait ever
// ran out, it sets kStatusSplitWait there (the sum is then incomplete and the
// host learns of it from qlora_device_status).
template <int NA, int NB, int NT = 256>
__device__ __forceinline__ bool splitk_combine(f32x16 (&acc)[NA][NB], float* __restrict__ slots, int* ticket,
                                               int* published, int S, int sidx, int* flag, int* status) {
  static_assert(NA * NB * 16 * NT == kSplitSlotFloats, "tile size");
  const int tid = threadIdx.x;
  const rsrc_t rs = make_rsrc(slots, (int64_t)S * kSplitSlotFloats * 4);
  __syncthreads();  // flag is free
  if (tid == 0) *flag = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  if (*flag != S - 1) {
    const uint32_t mine = (uint32_t)sidx * kSplitSlotFloats * 4;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint32_t off = (uint32_t)((((a * NB + b) * 4 + e4) * NT + tid) * 16);
          const u32x4 v = u32x4{__float_as_uint(acc[a][b][4 * e4]), __float_as_uint(acc[a][b][4 * e4 + 1]),
                                __float_as_uint(acc[a][b][4 * e4 + 2]), __float_as_uint(acc[a][b][4 * e4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), rs, (int)(mine + off), 0,
              kCachePolicySystem);
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's slot stores are complete
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(published, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return false;
  }
  // The others hold earlier tickets: they are past their main loops and
  // only store and publish.  The bound is a guard that is never reached; if
  // it were, the status word records it.
  if (tid == 0) {
    bool done = false;
    for (int spin = 0; spin < (1 << 24) && !done; ++spin) {
      done = __hip_atomic_load(published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >= S - 1;
      if (!done) __builtin_amdgcn_s_sleep(2);
    }
    if (!done) __hip_atomic_fetch_or(status, kStatusSplitWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __syncthreads();
  splitk_add_slots<3, 8>(acc, rs, S, sidx);
  if (tid == 0) {
    __hip_atomic_exchange(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_exchange(published, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  return true;
}

// Work plan of a tile grid on the 8 XCDs x 32 compute units.  Workgroup b
// runs on XCD b % 8; XCD x owns the contiguous tiles [x*tx, x*tx + tx).  Its
// first `full` tiles run whole; when the rest would fill at most half of the
// XCD's units in a last round, each of them is cut into S contraction slices
// so that the last round finishes sooner.  Items of an XCD are numbered in
// dispatch order (whole tiles first), slices of a tile adjacent.
struct SplitPlan {
  int tiles;      // real tiles
  int tx;         // tiles per XCD
  int full;       // whole tiles per XCD
  int S;          // slices of each remaining tile (1: none)
  int items;      // items per XCD
  int steps;      // contraction steps of a tile
  int steps_per;  // contraction steps of a slice
  __host__ __device__ int nsplit() const { return 8 * (tx - full); }  // split tiles, including any past `tiles`
};

inline SplitPlan make_split_plan(int64_t tiles, int64_t steps) {
  SplitPlan pl{};
  pl.tiles = (int)tiles;
  pl.steps = (int)steps;
  pl.tx = (int)((tiles + 7) / 8);
  const int rem = pl.tx <= 32 ? pl.tx : pl.tx % 32;
  pl.full = pl.tx - rem;
  pl.S = 1;
  if (rem > 0 && rem <= 16) {
    for (int S = 2; S <= 4; ++S) {
      if (rem * S > 32 || S > steps) break;
      if ((steps + S - 1) / S * (S - 1) >= steps) continue;  // no empty slice
      pl.S = S;
    }
  }
  if (pl.S == 1) pl.full = pl.tx;
  pl.items = pl.full + (pl.tx - pl.full) * pl.S;
  pl.steps_per = (int)((steps + pl.S - 1) / pl.S);
  return pl;
}

struct TileItem {
  int tile;     // tile index, or -1: nothing to do
  int sidx;     // slice
  int S;        // slices of this tile
  int ordinal;  // index among split tiles (slots / counter), -1 when whole
  int kbeg, kend;
};

__device__ __forceinline__ TileItem decode_item(const SplitPlan& pl, int bid) {
  TileItem it;
  const int xcd = bid & 7, local = bid >> 3;
  it.tile = -1;
  if (local >= pl.items) return it;
  if (local < pl.full) {
    it.tile = xcd * pl.tx + local;
    it.sidx = 0;
    it.S = 1;
    it.ordinal = -1;
    it.kbeg = 0;
    it.kend = pl.steps;
  } else {
    const int idx = local - pl.full;
    it.tile = xcd * pl.tx + pl.full + idx / pl.S;
    it.sidx = idx % pl.S;
    it.S = pl.S;
    it.ordinal = xcd * (pl.tx - pl.full) + idx / pl.S;
    it.kbeg = it.sidx * pl.steps_per;
    it.kend = it.kbeg + pl.steps_per < pl.steps ? it.kbeg + pl.steps_per : pl.steps;
  }
  if (it.tile >= pl.tiles) it.tile = -1;
  return it;
}

}  // namespace qlora
