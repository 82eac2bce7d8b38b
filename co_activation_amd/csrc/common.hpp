// Shared device helpers for the dispatch engine (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_coact.h"

namespace moe {

constexpr int kWave = 64;

// One launch holds fewer than 2^32 work-items: the dispatch packet counts a
// grid's work-items in 32 bits.  Launchers whose grid grows with rows times
// row width check this and refuse larger inputs with MOE_ERR_SHAPE.
inline bool grid_ok(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= INT32_MAX && blocks * threads < (int64_t{1} << 32);
}

// Launch-status check used right after every kernel launch.
#define MOE_CHECK_LAUNCH()                                  \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave index inside the block, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `m` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ long long wave_sum64(long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, kWave));
  return v;
}

// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

// Inclusive prefix max across the 64 lanes.
__device__ __forceinline__ int wave_incl_max(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v = max(v, u);
  }
  return v;
}

__device__ __forceinline__ void report(int32_t* d_err, int bits) {
  if (d_err != nullptr && bits != 0) atomicOr(d_err, bits);
}

}  // namespace moe
