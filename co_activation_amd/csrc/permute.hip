// Row scatter into rank-contiguous send buffers: the dispatched hidden
// states of "Training Communication-Efficient Mixture-of-Experts Language
// Models with Layer Re-Configuration" (footnote 3), sent once per destination
// rank as in "Expert Coupling in MoE Pretraining ..." (abstract); the same
// kernel moves tokens for the token shuffle.
//
// Token-major: one wave owns one token, reads its row once and writes it to
// each of its (<= 8) destination rows.  The destination list is wave-uniform
// and lives in scalar registers; each store instruction of the wave writes
// 64 x 16 contiguous bytes.  HBM-bound: algorithmic bytes per token are
// row_bytes * (1 + destinations) + 4 * width.
#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;

template <typename V, int UNROLL>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const V* __restrict__ x, int T, int64_t vec_per_row, const int32_t* __restrict__ dest,
    int width, V* __restrict__ out, int64_t out_rows, int32_t* d_err) {
  const int lane = lane_id();
  const int t = blockIdx.x * kPermWaves + wave_id();
  if (t >= T) return;

  // Destination rows (wave-uniform); -1 marks an absent or rejected one.
  int drow[MOE_MAX_K];
  int nd = 0;
  int errbits = 0;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    drow[q] = -1;
    if (q < width) {
      const int r = __builtin_amdgcn_readfirstlane(dest[static_cast<int64_t>(t) * width + q]);
      if (r >= 0 && r < out_rows) {
        drow[q] = r;
        ++nd;
      } else if (r >= out_rows) {
        errbits = MOE_DERR_ROW_RANGE;
      }
    }
  }
  if (lane == 0) report(d_err, errbits);
  if (nd == 0) return;

  const V* src = x + static_cast<int64_t>(t) * vec_per_row;
  for (int64_t c0 = lane; c0 < vec_per_row; c0 += kWave * UNROLL) {
    V v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < vec_per_row) v[u] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q) {
      if (q >= width) break;
      if (drow[q] < 0) continue;
      V* dst = out + static_cast<int64_t>(drow[q]) * vec_per_row;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t c = c0 + u * kWave;
        if (c < vec_per_row) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_permute(const void* x, int64_t T, int64_t row_bytes, const int32_t* dest,
                           int width, void* out, int64_t out_rows, int32_t* d_err, void* stream) {
  if (T < 0 || row_bytes <= 0 || width < 1 || width > MOE_MAX_K || out_rows < 0 ||
      T * static_cast<int64_t>(width) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || dest == nullptr || out == nullptr) return MOE_ERR_NULL;
  const auto xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
  if (row_bytes % 4 != 0 || xa % 4 != 0 || oa % 4 != 0) return MOE_ERR_ALIGN;
  const unsigned blocks = static_cast<unsigned>((T + moe::kPermWaves - 1) / moe::kPermWaves);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (row_bytes % 16 == 0 && xa % 16 == 0 && oa % 16 == 0) {
    moe::permute_kernel<moe::u32x4, 4><<<blocks, moe::kPermThreads, 0, s>>>(
        static_cast<const moe::u32x4*>(x), static_cast<int>(T), row_bytes / 16, dest, width,
        static_cast<moe::u32x4*>(out), out_rows, d_err);
  } else {
    moe::permute_kernel<uint32_t, 4><<<blocks, moe::kPermThreads, 0, s>>>(
        static_cast<const uint32_t*>(x), static_cast<int>(T), row_bytes / 4, dest, width,
        static_cast<uint32_t*>(out), out_rows, d_err);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
