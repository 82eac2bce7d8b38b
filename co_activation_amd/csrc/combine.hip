// Weighted combine back to token order: the hidden-state combine of
// "Training Communication-Efficient Mixture-of-Experts Language Models with
// Layer Re-Configuration" (footnote 3) over the rows of the deduplicated
// dispatch of "Expert Coupling in MoE Pretraining ..." (abstract).
//
//   y[t] = sum_q a(row_q) * z[row_q],  q over the token's rows in order,
//
// fp32 fused multiply-adds in ascending q, one rounding to the output type
// (bf16: round to nearest even).  A wave owns a chunk of one token's output
// row; the token's row list and weights are uniform (scalar registers); each
// lane owns groups of 8 (or 4 for fp32 -> fp32) consecutive elements,
// 16-byte nontemporal loads and stores.
// HBM-bound: algorithmic bytes per token are rows * (z row bytes + 4) +
// y row bytes + 4 * k.
#include "rowio.hpp"

namespace moe {
namespace {

constexpr int kCombThreads = 256;

// One wave per (token, chunk of kWave * U element groups): a row is split
// into chunks of U groups per lane, and each chunk of each token is an
// independent work item (four per 256-thread block).  The token's row list
// and weights are read per wave into scalar registers.
template <bool ZBF16, bool YBF16, int EPL, int U>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const u32x4* __restrict__ z, int64_t z_rows, int64_t groups, int chunks,
    const int32_t* __restrict__ rows, int k, const float* __restrict__ weight, int T,
    u32x4* __restrict__ y, const int32_t* __restrict__ n_valid, int32_t* d_err) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kCombThreads / kWave) + wave_id();
  const int t = static_cast<int>(item / chunks);
  if (t >= T || (n_valid != nullptr && t >= *n_valid)) return;
  const int chunk = static_cast<int>(item - static_cast<int64_t>(t) * chunks);
  const int lane = lane_id();

  // 16-byte vectors per row of z and of y.
  const int64_t zvec = groups * (ZBF16 ? EPL / 8 : EPL / 4);
  const int64_t yvec = groups * (YBF16 ? EPL / 8 : EPL / 4);

  // The token's rows, then their weights: every load of a kind is issued
  // before any is used, so the prologue costs two memory latencies.
  int rid[MOE_MAX_K];
  float a[MOE_MAX_K];
  int errbits = 0;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q)
    rid[q] = q < k ? __builtin_amdgcn_readfirstlane(rows[static_cast<int64_t>(t) * k + q]) : -1;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    if (rid[q] >= z_rows) {
      errbits = MOE_DERR_ROW_RANGE;
      rid[q] = -1;
    }
  }
  if (weight != nullptr && z_rows > 0) {
    // One load per slot, absent rows reading row 0's weight (unused).
    float wv[MOE_MAX_K];
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q) wv[q] = weight[rid[q] < 0 ? 0 : rid[q]];
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q)
      a[q] = rid[q] < 0 ? 0.f : __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wv[q])));
  } else {
#pragma unroll
    for (int q = 0; q < MOE_MAX_K; ++q) a[q] = rid[q] < 0 ? 0.f : 1.f;
  }
  if (chunk == 0 && lane == 0) report(d_err, errbits);

  u32x4* yrow = y + static_cast<int64_t>(t) * yvec;
  const int64_t g0 = static_cast<int64_t>(chunk) * (kWave * U) + lane;
  float acc[U][EPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[u][i] = 0.f;
#pragma unroll
  for (int q = 0; q < MOE_MAX_K; ++q) {
    if (q >= k) break;
    if (rid[q] < 0) continue;
    const u32x4* zrow = z + static_cast<int64_t>(rid[q]) * zvec;
    float f[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u * kWave;
      if (g < groups) load_group<ZBF16, EPL>(zrow, g, f[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[u][i] = __builtin_fmaf(a[q], f[u][i], acc[u][i]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + u * kWave;
    if (g < groups) store_group<YBF16, EPL>(yrow, g, acc[u]);
  }
}

// Tokens with many rows (k >= 6 slots and at least 6 rows of z per output
// row, so that most slots are in use -- not so for the expert side's reply
// rows, whose k slots hold one or two rows): blocks reserve LDS they do not
// use, to cap how many are resident per CU (160 KB of LDS).  Measured on
// MI355X:
//  - rows of at most 8 KiB: one group per lane (1 KiB of each row per wave)
//    and at most eight blocks per CU; k = 6 with 8 KiB rows combines in 460
//    us inside the one-layer step against 480 with two groups per lane and
//    six blocks (466 against 507 alone);
//  - wider rows: two groups per lane and at most six blocks per CU; k = 8
//    with 14 KiB rows in 635 us inside the step against 651 with one group
//    and eight blocks, and against 667 with no cap;
//  - one or two rows per output row: two groups per lane and no cap (k = 2:
//    240 us against 272 with one group; the cap costs 8-14% there).
constexpr unsigned kCombLdsNarrow = 20 * 1024;  // eight blocks per CU
constexpr unsigned kCombLdsWide = 24 * 1024;    // six blocks per CU

template <bool ZBF16, bool YBF16, int EPL, int U>
int launch_u(const void* z, int64_t z_rows, int64_t H, const int32_t* rows, int k, const float* w,
             int64_t T, void* y, const int32_t* n_valid, int32_t* d_err, unsigned lds,
             hipStream_t s) {
  const int64_t groups = H / EPL;
  const int chunks = static_cast<int>((groups + kWave * U - 1) / (kWave * U));
  const int64_t items = T * chunks;
  constexpr int kItemsPerBlock = kCombThreads / kWave;
  const int64_t blocks = (items + kItemsPerBlock - 1) / kItemsPerBlock;
  if (!grid_ok(blocks, kCombThreads)) return MOE_ERR_SHAPE;
  combine_kernel<ZBF16, YBF16, EPL, U><<<static_cast<unsigned>(blocks), kCombThreads, lds, s>>>(
      static_cast<const u32x4*>(z), z_rows, groups, chunks, rows, k, w, static_cast<int>(T),
      static_cast<u32x4*>(y), n_valid, d_err);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <bool ZBF16, bool YBF16, int EPL>
int launch(const void* z, int64_t z_rows, int64_t H, const int32_t* rows, int k, const float* w,
           int64_t T, void* y, const int32_t* n_valid, int32_t* d_err, hipStream_t s) {
  const bool many = k >= 6 && z_rows >= 6 * T;
  const int64_t z_row_bytes = H * (ZBF16 ? 2 : 4);
  if (many && z_row_bytes <= 8192)
    return launch_u<ZBF16, YBF16, EPL, 1>(z, z_rows, H, rows, k, w, T, y, n_valid, d_err,
                                          kCombLdsNarrow, s);
  return launch_u<ZBF16, YBF16, EPL, 2>(z, z_rows, H, rows, k, w, T, y, n_valid, d_err,
                                        many ? kCombLdsWide : 0u, s);
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine(const void* z, int z_dtype, int64_t z_rows, int64_t H,
                           const int32_t* rows, int k, const float* row_weight, int64_t T,
                           void* y, int y_dtype, const int32_t* n_valid, int32_t* d_err,
                           void* stream) {
  if ((z_dtype != MOE_F32 && z_dtype != MOE_BF16) || (y_dtype != MOE_F32 && y_dtype != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (T < 0 || H <= 0 || z_rows < 0 || k < 1 || k > MOE_MAX_K ||
      T * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (z == nullptr || rows == nullptr || y == nullptr) return MOE_ERR_NULL;
  const int zb = z_dtype == MOE_BF16 ? 2 : 4, yb = y_dtype == MOE_BF16 ? 2 : 4;
  if ((H * zb) % 16 != 0 || (H * yb) % 16 != 0 || reinterpret_cast<uintptr_t>(z) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(y) % 16 != 0)
    return MOE_ERR_ALIGN;
  if (moe::overlap(z, z_rows * H * zb, y, T * H * yb)) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (z_dtype == MOE_BF16 && y_dtype == MOE_BF16)
    return moe::launch<true, true, 8>(z, z_rows, H, rows, k, row_weight, T, y, n_valid, d_err, s);
  if (z_dtype == MOE_BF16 && y_dtype == MOE_F32)
    return moe::launch<true, false, 8>(z, z_rows, H, rows, k, row_weight, T, y, n_valid, d_err, s);
  if (z_dtype == MOE_F32 && y_dtype == MOE_BF16)
    return moe::launch<false, true, 8>(z, z_rows, H, rows, k, row_weight, T, y, n_valid, d_err, s);
  return moe::launch<false, false, 4>(z, z_rows, H, rows, k, row_weight, T, y, n_valid, d_err, s);
}
