// Element-group row I/O shared by the kernels that compute on row values
// (combine, scaled scatter, row dot): 16-byte nontemporal accesses, bf16 or
// fp32 elements, groups of EPL consecutive elements.
#pragma once

#include "common.hpp"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// EPL elements of one row starting at element group g.
template <bool ZBF16, int EPL>
__device__ __forceinline__ void load_group(const u32x4* __restrict__ row, int64_t g, float (&f)[EPL]) {
  if constexpr (ZBF16) {
    static_assert(EPL == 8, "bf16 groups are 8 elements");
    const u32x4 v = __builtin_nontemporal_load(row + g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < EPL / 4; ++h) {
      const u32x4 v = __builtin_nontemporal_load(row + g * (EPL / 4) + h);
#pragma unroll
      for (int i = 0; i < 4; ++i) f[4 * h + i] = __uint_as_float(v[i]);
    }
  }
}

template <bool YBF16, int EPL>
__device__ __forceinline__ void store_group(u32x4* __restrict__ row, int64_t g, const float (&f)[EPL]) {
  if constexpr (YBF16) {
    static_assert(EPL == 8, "bf16 groups are 8 elements");
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = to_bf16(f[2 * i]) | (to_bf16(f[2 * i + 1]) << 16);
    __builtin_nontemporal_store(v, row + g);
  } else {
#pragma unroll
    for (int h = 0; h < EPL / 4; ++h) {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[4 * h + i]);
      __builtin_nontemporal_store(v, row + g * (EPL / 4) + h);
    }
  }
}


}  // namespace moe
