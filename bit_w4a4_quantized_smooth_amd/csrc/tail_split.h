// The split last round of a 128 x 128-tile GEMM grid (both 4-bit GEMMs): the
// mapping of a workgroup to its tile and K slice, and the exchange of the
// slices' fp32 partial accumulators through the caller's workspace.
#pragma once

#include "common.h"
#include "launch.h"

namespace svdq {

// Tile index t in the XCD-contiguous order of a grid of `tiles` tiles (a
// multiple of 8) for workgroup b; for the workgroups past ts.full, also the
// K slice and the index of the split tile (slice stays -1 otherwise).
// Whole tiles are the first tpx - tail/8 of each XCD's range of tpx = tiles/8,
// the split tiles its last tail/8; the slices of a split tile are dispatched
// to the same XCD (workgroup ids congruent mod 8).
__device__ __forceinline__ int split_tile_of(int b, int tiles, const TailSplit& ts, int& slice, int& tail_idx) {
  const int tpx = tiles >> 3;
  slice = -1;
  tail_idx = 0;
  if (ts.parts > 0 && b >= ts.full) {
    const int sb = b - ts.full, tail_px = ts.tail >> 3, j = sb >> 3;
    const int tt = j % tail_px;
    slice = j / tail_px;
    tail_idx = (sb & 7) * tail_px + tt;
    return (sb & 7) * tpx + (tpx - tail_px) + tt;
  }
  return (b & 7) * tpx + (b >> 3);
}

// A K slice's end: store this workgroup's partial accumulators (NV 4-float
// vectors per lane, four waves) with agent-coherent stores, wait until they
// are performed, count the slice in; the last slice of the tile to arrive
// resets the counter and replaces its accumulators with the sum of all
// slices' partials in slice order (the same sum whichever slice it is) and
// returns true; the others return false and end.  `flag` is a word of LDS
// that no wave still reads.  No workgroup waits for another.
template <int NV, class Get, class Set>
__device__ __forceinline__ bool split_exchange(const TailSplit& ts, int tail_idx, int slice, int wave, int lane,
                                               int tid, unsigned* flag, Get get, Set set) {
  constexpr int PER = 4 * NV * 64 * 4;  // floats of one partial tile
  static_assert((size_t)PER * 4 == kTailTileBytes, "partial tile size");
  float* const base = ts.part + (size_t)tail_idx * ts.parts * PER;
  // layout [wave][vector][half][lane] of 8-byte words: each store instruction
  // writes 512 contiguous bytes (whole lines)
  uint64_t* const mine = (uint64_t*)(base + (size_t)slice * PER) + (size_t)wave * NV * 128 + lane;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint4 v = __builtin_bit_cast(uint4, get(k));
    __hip_atomic_store(mine + k * 128, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + k * 128 + 64, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // every store of this wave performed
  __syncthreads();
  if (tid == 0) *flag = __hip_atomic_fetch_add(ts.cnt + tail_idx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned arrived = __builtin_amdgcn_readfirstlane(*(volatile unsigned*)flag);
  if (arrived != (unsigned)ts.parts - 1) return false;
  if (tid == 0) __hip_atomic_store(ts.cnt + tail_idx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v4f sum[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) sum[k] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < ts.parts; ++q) {
    const uint64_t* const src = (const uint64_t*)(base + (size_t)q * PER) + (size_t)wave * NV * 128 + lane;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      v4f p = get(k);
      if (q != slice) {
        const uint64_t lo = __hip_atomic_load(src + k * 128, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi = __hip_atomic_load(src + k * 128 + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p = __builtin_bit_cast(v4f, uint4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)});
      }
      sum[k] += p;
    }
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) set(k, sum[k]);
  return true;
}

}  // namespace svdq
