// Co-activation statistics of one MoE layer.
//
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training" (Key Observation): the set of tokens that activate each expert
// and the Ochiai similarity |A n B| / sqrt(|A| |B|) of two experts.
// "Expert Coupling in MoE Pretraining ..." (abstract): expert pairs selected
// together in a layer, and the experts of one layer predicting those of the
// next (transition counts).
//
// Each block owns a slice of matrix rows as a 64 KB LDS histogram and a
// chunk of tokens; every token adds its slot pairs with LDS atomics; the
// non-zero bins are then added to the output with global atomics.  Integer
// addition is associative, so the counts do not depend on scheduling.  The
// pair matrix is counted on and above the diagonal only (i <= j, the
// diagonal being the per-expert count); a final pass mirrors it, copies the
// diagonal out and evaluates Ochiai in double precision.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kStatThreads = 256;
constexpr int kHistBins = 16384;  // 64 KB of int32 per block
constexpr int kTokensPerBlock = 1024;

enum StatMode { kCounts = 0, kPairs = 1, kTransitions = 2 };

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// Reads one token's ids into e[]; out-of-range slots become -1.
__device__ __forceinline__ int load_ids(const int32_t* __restrict__ row, int k, int E,
                                        int (&e)[MOE_MAX_K]) {
  int err = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    e[j] = -1;
    if (j < k) {
      const int v = row[j];
#pragma unroll
      for (int q = 0; q < j; ++q)
        if (e[q] == v && v >= 0 && v < E) err |= MOE_DERR_EXPERT_DUP;
      if (v >= 0 && v < E)
        e[j] = v;
      else
        err |= MOE_DERR_EXPERT_RANGE;
    }
  }
  return err;
}

// MODE kCounts: bins = experts.  kPairs: bins = (i, j), i <= j, rows of the
// slice.  kTransitions: bins = (i in this layer, j in the next layer).
template <int MODE>
__global__ __launch_bounds__(kStatThreads) void stats_count_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int32_t* __restrict__ topk2,
    int k2, int E2, int ncols, int rows_per_slice, int nrows, int tokens_per_block,
    int32_t* __restrict__ out, int32_t* d_err, int report_errors) {
  __shared__ int hist[kHistBins];
  const int r0 = blockIdx.y * rows_per_slice;
  const int r1 = min(r0 + rows_per_slice, nrows);
  const int slice_bins = (r1 - r0) * ncols;
  for (int i = threadIdx.x; i < slice_bins; i += kStatThreads) hist[i] = 0;
  __syncthreads();

  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(T, tb0 + tokens_per_block);
  int errbits = 0;
  for (int t = tb0 + static_cast<int>(threadIdx.x); t < tb1; t += kStatThreads) {
    int e[MOE_MAX_K];
    errbits |= load_ids(topk + static_cast<int64_t>(t) * k, k, E, e);
    if constexpr (MODE == kCounts) {
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a)
        if (a < k && e[a] >= 0) atomicAdd(&hist[e[a]], 1);
    } else if constexpr (MODE == kPairs) {
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a) {
        if (a >= k || e[a] < 0) continue;
#pragma unroll
        for (int b = a; b < MOE_MAX_K; ++b) {
          if (b >= k || e[b] < 0) continue;
          const int i = min(e[a], e[b]), j = max(e[a], e[b]);
          if (i >= r0 && i < r1) atomicAdd(&hist[(i - r0) * ncols + j], 1);
        }
      }
    } else {
      int f[MOE_MAX_K];
      errbits |= load_ids(topk2 + static_cast<int64_t>(t) * k2, k2, E2, f);
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a) {
        if (a >= k || e[a] < r0 || e[a] >= r1) continue;
#pragma unroll
        for (int b = 0; b < MOE_MAX_K; ++b)
          if (b < k2 && f[b] >= 0) atomicAdd(&hist[(e[a] - r0) * ncols + f[b]], 1);
      }
    }
  }
  if (report_errors && blockIdx.y == 0) report(d_err, errbits);
  __syncthreads();
  int32_t* dst = out + static_cast<int64_t>(r0) * ncols;
  for (int i = threadIdx.x; i < slice_bins; i += kStatThreads) {
    const int v = hist[i];
    if (v != 0) atomicAdd(dst + i, v);
  }
}

// Mirror the counted upper triangle, copy out the diagonal, Ochiai.
__global__ void stats_finish_kernel(int E, int32_t* __restrict__ pair_count,
                                    int32_t* __restrict__ expert_count, float* __restrict__ ochiai) {
  const int64_t n = static_cast<int64_t>(E) * E;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(idx / E), j = static_cast<int>(idx - static_cast<int64_t>(i) * E);
    const int c = i <= j ? pair_count[idx] : pair_count[static_cast<int64_t>(j) * E + i];
    if (i > j) pair_count[idx] = c;
    if (i == j) expert_count[i] = c;
    if (ochiai != nullptr) {
      const int ni = pair_count[static_cast<int64_t>(i) * E + i];
      const int nj = pair_count[static_cast<int64_t>(j) * E + j];
      const double d = static_cast<double>(ni) * static_cast<double>(nj);
      ochiai[idx] = d > 0.0 ? static_cast<float>(static_cast<double>(c) / sqrt(d)) : 0.f;
    }
  }
}

int launch_fill(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  const int64_t blocks = (n + 255) / 256;
  fill_zero_kernel<<<static_cast<unsigned>(blocks < 1024 ? blocks : 1024), 256, 0, s>>>(p, n);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <int MODE>
int launch_count(const int32_t* topk, int T, int k, int E, const int32_t* topk2, int k2, int E2,
                 int32_t* out, int32_t* d_err, int report_errors, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int ncols = MODE == kCounts ? E : (MODE == kPairs ? E : E2);
  const int nrows = MODE == kCounts ? 1 : E;
  const int rows_per_slice = MODE == kCounts ? 1 : kHistBins / ncols;
  const int slices = (nrows + rows_per_slice - 1) / rows_per_slice;
  const int bx = (T + kTokensPerBlock - 1) / kTokensPerBlock;
  stats_count_kernel<MODE><<<dim3(bx, slices), kStatThreads, 0, s>>>(
      topk, T, k, E, topk2, k2, E2, ncols, rows_per_slice, nrows, kTokensPerBlock, out, d_err,
      report_errors);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_coact_stats(const int32_t* topk, int64_t T, int k, int E,
                               const int32_t* topk_next, int k_next, int E_next,
                               int32_t* expert_count, int32_t* pair_count, float* ochiai,
                               int32_t* transition, int32_t* d_err, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_E ||
      T * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (transition != nullptr &&
      (k_next < 1 || k_next > MOE_MAX_K || E_next < 1 || E_next > MOE_MAX_E ||
       T * static_cast<int64_t>(k_next) >= (int64_t{1} << 31)))
    return MOE_ERR_SHAPE;
  if (expert_count == nullptr) return MOE_ERR_NULL;
  if (ochiai != nullptr && pair_count == nullptr) return MOE_ERR_NULL;
  if (T > 0 && topk == nullptr) return MOE_ERR_NULL;
  if (transition != nullptr && T > 0 && topk_next == nullptr) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);
  int st;
  if (pair_count != nullptr) {
    if ((st = moe::launch_fill(pair_count, static_cast<int64_t>(E) * E, s)) != MOE_OK) return st;
    if ((st = moe::launch_count<moe::kPairs>(topk, Ti, k, E, nullptr, 0, 0, pair_count, d_err, 1,
                                             s)) != MOE_OK)
      return st;
    const int64_t n = static_cast<int64_t>(E) * E;
    const int64_t blocks = (n + 255) / 256;
    moe::stats_finish_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(E, pair_count,
                                                                           expert_count, ochiai);
    MOE_CHECK_LAUNCH();
  } else {
    if ((st = moe::launch_fill(expert_count, E, s)) != MOE_OK) return st;
    if ((st = moe::launch_count<moe::kCounts>(topk, Ti, k, E, nullptr, 0, 0, expert_count, d_err,
                                              1, s)) != MOE_OK)
      return st;
  }
  if (transition != nullptr) {
    if ((st = moe::launch_fill(transition, static_cast<int64_t>(E) * E_next, s)) != MOE_OK)
      return st;
    if ((st = moe::launch_count<moe::kTransitions>(topk, Ti, k, E, topk_next, k_next, E_next,
                                                   transition, d_err, 1, s)) != MOE_OK)
      return st;
  }
  return MOE_OK;
}
