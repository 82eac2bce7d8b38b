// Shared device helpers for the dispatch engine (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
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

// True when the byte ranges [a, a + a_bytes) and [b, b + b_bytes) share a
// byte (an output that overlaps an input: blocks would read rows that
// others have already overwritten).
inline bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (a == nullptr || b == nullptr || a_bytes <= 0 || b_bytes <= 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(b_bytes) && pb < pa + static_cast<uintptr_t>(a_bytes);
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


// Sum over the 64 lanes, every lane receiving it: the DPP inclusive scan of
// wave_incl_scan on 64-bit values (each half moved separately), then lane
// 63's total.
__device__ __forceinline__ long long wave_sum64(long long v) {
  const int lane = lane_id();
  const int rl = lane & 15;
  auto mv = [](long long x, auto ctrl) {
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<unsigned long long>(x)),
                                               decltype(ctrl)::value, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<unsigned long long>(x) >> 32),
                                               decltype(ctrl)::value, 0xF, 0xF, false);
    return static_cast<long long>((static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
                                  static_cast<uint32_t>(lo));
  };
  long long t = mv(v, std::integral_constant<int, 0x111>{});  // row_shr:1
  if (rl >= 1) v += t;
  t = mv(v, std::integral_constant<int, 0x112>{});  // row_shr:2
  if (rl >= 2) v += t;
  t = mv(v, std::integral_constant<int, 0x114>{});  // row_shr:4
  if (rl >= 4) v += t;
  t = mv(v, std::integral_constant<int, 0x118>{});  // row_shr:8
  if (rl >= 8) v += t;
  t = mv(v, std::integral_constant<int, 0x142>{});  // row_bcast:15
  if ((lane & 31) >= 16) v += t;
  t = mv(v, std::integral_constant<int, 0x143>{});  // row_bcast:31
  if (lane >= 32) v += t;
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned long long>(v)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned long long>(v) >> 32), 63);
  return static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo);
}


// Lane `src`'s value of v, for a src that is the same in every lane.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}

// Inclusive prefix sum across the 64 lanes, with DPP lane moves instead of
// LDS permutes: shifts by 1, 2, 4 and 8 lanes inside each row of 16, then
// lane 15 of a row broadcast into the next row (row_bcast:15, added in rows
// 1 and 3) and lane 31 into the upper half (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
  const int rl = lane & 15;
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  if (rl >= 1) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  if (rl >= 2) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  if (rl >= 4) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  if (rl >= 8) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xF, 0xF, false);  // row_bcast:15
  if ((lane & 31) >= 16) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xF, 0xF, false);  // row_bcast:31
  if (lane >= 32) v += t;
  return v;
}

// Inclusive prefix max across the 64 lanes (the same lane moves).
__device__ __forceinline__ int wave_incl_max(int v) {
  const int lane = lane_id();
  const int rl = lane & 15;
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  if (rl >= 1) v = max(v, t);
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  if (rl >= 2) v = max(v, t);
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  if (rl >= 4) v = max(v, t);
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  if (rl >= 8) v = max(v, t);
  t = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xF, 0xF, false);
  if ((lane & 31) >= 16) v = max(v, t);
  t = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xF, 0xF, false);
  if (lane >= 32) v = max(v, t);
  return v;
}

// Sum and maximum over the 64 lanes, every lane receiving them: lane 63 of
// the inclusive scan.
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

__device__ __forceinline__ int wave_max(int v) {
  return __builtin_amdgcn_readlane(wave_incl_max(v), 63);
}

// Segmented inclusive prefix sum across the 64 lanes: a lane whose flag is
// set starts a new segment.  The combine of (value, flag) pairs -- a later
// pair that starts a segment keeps its value, otherwise it adds the earlier
// one; flags or together -- is associative, so the DPP steps of
// wave_incl_scan apply.  On return flag says whether a segment starts at or
// before the lane.
__device__ __forceinline__ void wave_seg_scan(int& val, int& flag) {
  const int lane = lane_id();
  const int rl = lane & 15;
#define MOE_SEG_STEP(CTRL, COND)                                             \
  {                                                                          \
    const int uv = __builtin_amdgcn_update_dpp(0, val, CTRL, 0xF, 0xF, false); \
    const int uf = __builtin_amdgcn_update_dpp(0, flag, CTRL, 0xF, 0xF, false); \
    if (COND) {                                                              \
      if (!flag) val += uv;                                                  \
      flag |= uf;                                                            \
    }                                                                        \
  }
  MOE_SEG_STEP(0x111, rl >= 1)             // row_shr:1
  MOE_SEG_STEP(0x112, rl >= 2)             // row_shr:2
  MOE_SEG_STEP(0x114, rl >= 4)             // row_shr:4
  MOE_SEG_STEP(0x118, rl >= 8)             // row_shr:8
  MOE_SEG_STEP(0x142, (lane & 31) >= 16)   // row_bcast:15
  MOE_SEG_STEP(0x143, lane >= 32)          // row_bcast:31
#undef MOE_SEG_STEP
}

__device__ __forceinline__ void report(int32_t* d_err, int bits) {
  if (d_err != nullptr && bits != 0) atomicOr(d_err, bits);
}

}  // namespace moe
