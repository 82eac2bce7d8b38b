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

// Work of one statistics call, split into histogram slices of matrix rows:
// slices [0, a_slices) belong to matrix A (per-expert counts, or the pair
// matrix counted on and above its diagonal), slices [a_slices, a_slices +
// b_slices) to the transition matrix B.
struct StatsJob {
  int a_mode;  // kCounts or kPairs
  int a_rows, a_cols, a_rps, a_slices;
  int32_t* a_out;
  int b_rows, b_cols, b_rps, b_slices;
  int32_t* b_out;
};

// Zeroes the output arrays the count pass accumulates into.
__global__ void zero_kernel(int32_t* __restrict__ a, int64_t na, int32_t* __restrict__ b, int64_t nb) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < na + nb;
       i += stride) {
    if (i < na)
      a[i] = 0;
    else
      b[i - na] = 0;
  }
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

__global__ __launch_bounds__(kStatThreads) void stats_count_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int32_t* __restrict__ topk2,
    int k2, int E2, StatsJob job, int tokens_per_block, int32_t* d_err) {
  __shared__ int hist[kHistBins];
  const int slice = blockIdx.y;
  const bool in_a = slice < job.a_slices;
  const int mode = in_a ? job.a_mode : kTransitions;
  const int rps = in_a ? job.a_rps : job.b_rps;
  const int nrows = in_a ? job.a_rows : job.b_rows;
  const int ncols = in_a ? job.a_cols : job.b_cols;
  const int r0 = (in_a ? slice : slice - job.a_slices) * rps;
  const int r1 = min(r0 + rps, nrows);
  const int slice_bins = (r1 - r0) * ncols;
  for (int i = threadIdx.x; i < slice_bins; i += kStatThreads) hist[i] = 0;
  __syncthreads();

  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(T, tb0 + tokens_per_block);
  int errbits = 0;
  for (int t = tb0 + static_cast<int>(threadIdx.x); t < tb1; t += kStatThreads) {
    int e[MOE_MAX_K];
    errbits |= load_ids(topk + static_cast<int64_t>(t) * k, k, E, e);
    if (mode == kCounts) {
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a)
        if (a < k && e[a] >= 0) atomicAdd(&hist[e[a]], 1);
    } else if (mode == kPairs) {
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
  // One slice of each matrix reports the data errors it saw.
  if (slice == 0 || slice == job.a_slices) report(d_err, errbits);
  __syncthreads();
  int32_t* dst = (in_a ? job.a_out : job.b_out) + static_cast<int64_t>(r0) * ncols;
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

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 1024 ? 1024 : b));
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

  moe::StatsJob job{};
  if (pair_count != nullptr) {
    job.a_mode = moe::kPairs;
    job.a_rows = E;
    job.a_cols = E;
    job.a_rps = moe::kHistBins / E;
    job.a_out = pair_count;
  } else {
    job.a_mode = moe::kCounts;
    job.a_rows = 1;
    job.a_cols = E;
    job.a_rps = 1;
    job.a_out = expert_count;
  }
  job.a_slices = (job.a_rows + job.a_rps - 1) / job.a_rps;
  const int64_t na = static_cast<int64_t>(job.a_rows) * job.a_cols;
  int64_t nb = 0;
  if (transition != nullptr) {
    job.b_rows = E;
    job.b_cols = E_next;
    job.b_rps = moe::kHistBins / E_next;
    job.b_slices = (E + job.b_rps - 1) / job.b_rps;
    job.b_out = transition;
    nb = static_cast<int64_t>(E) * E_next;
  }

  moe::zero_kernel<<<moe::grid_for(na + nb), 256, 0, s>>>(job.a_out, na, job.b_out, nb);
  MOE_CHECK_LAUNCH();
  if (Ti > 0) {
    const int bx = (Ti + moe::kTokensPerBlock - 1) / moe::kTokensPerBlock;
    moe::stats_count_kernel<<<dim3(bx, job.a_slices + job.b_slices), moe::kStatThreads, 0, s>>>(
        topk, Ti, k, E, topk_next, k_next, E_next, job, moe::kTokensPerBlock, d_err);
    MOE_CHECK_LAUNCH();
  }
  if (pair_count != nullptr) {
    moe::stats_finish_kernel<<<moe::grid_for(static_cast<int64_t>(E) * E), 256, 0, s>>>(
        E, pair_count, expert_count, ochiai);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}

namespace moe {
namespace {

// state[i] = beta * state[i] + (1 - beta) * x[i]; the two products and the
// sum are rounded separately (no fused multiply-add), in that order.
__global__ void ema_kernel(float* __restrict__ state, const int32_t* __restrict__ x, int64_t n,
                           float beta, float one_minus_beta) {
#pragma clang fp contract(off)
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
    state[i] = state[i] * beta + static_cast<float>(x[i]) * one_minus_beta;
}

}  // namespace
}  // namespace moe

extern "C" int moe_ema_update(float* state, const int32_t* x, int64_t n, float beta,
                              void* stream) {
  if (n < 0 || !(beta >= 0.f && beta <= 1.f)) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (state == nullptr || x == nullptr) return MOE_ERR_NULL;
  const float omb = 1.f - beta;
  moe::ema_kernel<<<moe::grid_for(n), 256, 0, static_cast<hipStream_t>(stream)>>>(state, x, n, beta,
                                                                                  omb);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
