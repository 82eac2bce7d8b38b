// Co-activation statistics of one MoE layer.
//
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training" (Key Observation): the set of tokens that activate each expert
// and the Ochiai similarity |A n B| / sqrt(|A| |B|) of two experts.
// "Expert Coupling in MoE Pretraining ..." (abstract): expert pairs selected
// together in a layer, and the experts of one layer predicting those of the
// next (transition counts).
//
// The token range is cut into splits and the matrix rows into slices of at
// most kSliceBins bins; block (split, slice) counts its split's tokens into a
// 16 KB LDS histogram of its slice with LDS atomics and writes the histogram
// to its own partial row in the workspace (each thread loads the ids of its
// tokens of a pass before counting any, so their latencies overlap).  A sum
// kernel adds the splits' partials bin by bin (integer addition, so the
// counts do not depend on scheduling), and a finish kernel mirrors the pair
// matrix, copies the diagonal out as the per-expert counts and evaluates
// Ochiai in double precision.  No global atomics; every output element is written, so nothing
// needs clearing first.  The pair matrix is counted on and above the
// diagonal only (i <= j).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kStatThreads = 256;
constexpr int kSliceBins = 4096;         // 16 KB of int32 per block
constexpr int kTokensPerThread = 4;
constexpr int kSplitTokens = kStatThreads * kTokensPerThread;  // until kMaxSplits
constexpr int kMaxSplits = 64;

enum StatMode { kCounts = 0, kPairs = 1, kTransitions = 2 };

// Work of one statistics call.  Matrix A is the per-expert counts (one row
// of E bins) or the pair matrix (E x E, upper triangle counted); matrix B the
// transitions (E x E_next).  Slices [0, a_slices) cover A's rows, a_rps rows
// each; [a_slices, a_slices + b_slices) cover B's.  A split's partial row
// holds A's bins, then B's.
struct StatsJob {
  int a_mode;  // kCounts or kPairs
  int a_rows, a_cols, a_rps, a_slices;
  int b_rows, b_cols, b_rps, b_slices;
  int splits, split_tokens;
  int64_t a_bins, b_bins;  // bins of each matrix in a partial row
};

StatsJob stats_job(int64_t T, int E, bool pairs, bool transitions, int E_next) {
  StatsJob j{};
  j.a_mode = pairs ? kPairs : kCounts;
  j.a_rows = pairs ? E : 1;
  j.a_cols = E;
  j.a_rps = pairs ? kSliceBins / E : 1;
  j.a_slices = (j.a_rows + j.a_rps - 1) / j.a_rps;
  j.a_bins = static_cast<int64_t>(j.a_rows) * j.a_cols;
  if (transitions) {
    j.b_rows = E;
    j.b_cols = E_next;
    j.b_rps = kSliceBins / E_next;
    j.b_slices = (E + j.b_rps - 1) / j.b_rps;
    j.b_bins = static_cast<int64_t>(E) * E_next;
  }
  int64_t splits = (T + kSplitTokens - 1) / kSplitTokens;
  if (splits < 1) splits = 1;
  if (splits > kMaxSplits) splits = kMaxSplits;
  j.splits = static_cast<int>(splits);
  j.split_tokens = static_cast<int>((T + splits - 1) / splits);
  return j;
}

size_t stats_workspace_bytes(const StatsJob& j) {
  const size_t b = sizeof(int32_t) * static_cast<size_t>(j.splits) * (j.a_bins + j.b_bins);
  return (b + 255) & ~static_cast<size_t>(255);
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
    int k2, int E2, StatsJob job, int32_t* __restrict__ partial, int32_t* d_err) {
  __shared__ int hist[kSliceBins];
  const int split = blockIdx.x;
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

  const int tb0 = split * job.split_tokens;
  const int tb1 = min(T, tb0 + job.split_tokens);
  int errbits = 0;
  // kTokensPerThread tokens per pass, their ids loaded before any is counted
  for (int base = tb0; base < tb1; base += kStatThreads * kTokensPerThread) {
    int e[kTokensPerThread][MOE_MAX_K];
    int f[kTokensPerThread][MOE_MAX_K];
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
      const int t = base + u * kStatThreads + static_cast<int>(threadIdx.x);
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a) e[u][a] = f[u][a] = -1;
      if (t < tb1) {
        errbits |= load_ids(topk + static_cast<int64_t>(t) * k, k, E, e[u]);
        if (mode == kTransitions) errbits |= load_ids(topk2 + static_cast<int64_t>(t) * k2, k2, E2, f[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
      if (mode == kCounts) {
#pragma unroll
        for (int a = 0; a < MOE_MAX_K; ++a)
          if (a < k && e[u][a] >= 0) atomicAdd(&hist[e[u][a]], 1);
      } else if (mode == kPairs) {
#pragma unroll
        for (int a = 0; a < MOE_MAX_K; ++a) {
          if (a >= k || e[u][a] < 0) continue;
#pragma unroll
          for (int b = a; b < MOE_MAX_K; ++b) {
            if (b >= k || e[u][b] < 0) continue;
            const int i = min(e[u][a], e[u][b]), j = max(e[u][a], e[u][b]);
            if (i >= r0 && i < r1) atomicAdd(&hist[(i - r0) * ncols + j], 1);
          }
        }
      } else {
#pragma unroll
        for (int a = 0; a < MOE_MAX_K; ++a) {
          if (a >= k || e[u][a] < r0 || e[u][a] >= r1) continue;
#pragma unroll
          for (int b = 0; b < MOE_MAX_K; ++b)
            if (b < k2 && f[u][b] >= 0) atomicAdd(&hist[(e[u][a] - r0) * ncols + f[u][b]], 1);
        }
      }
    }
  }
  // One slice of each matrix reports the data errors it saw.
  if (slice == 0 || slice == job.a_slices) report(d_err, errbits);
  __syncthreads();
  int32_t* dst = partial + static_cast<int64_t>(split) * (job.a_bins + job.b_bins) +
                 (in_a ? 0 : job.a_bins) + static_cast<int64_t>(r0) * ncols;
  for (int i = threadIdx.x; i < slice_bins; i += kStatThreads) dst[i] = hist[i];
}

// Sum over the splits of one partial bin (independent loads, unrolled).
__device__ __forceinline__ int split_sum(const int32_t* __restrict__ p, int64_t row, int splits) {
  int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += p[static_cast<int64_t>(s + q) * row];
  }
  for (; s < splits; ++s) acc[0] += p[static_cast<int64_t>(s) * row];
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// Adds the splits' partials bin by bin: A's bins into pair_count (on and
// above the diagonal; the finish kernel fills the rest) or expert_count, B's
// into transition.
__global__ void stats_sum_kernel(const int32_t* __restrict__ partial, StatsJob job, int E,
                                 int32_t* __restrict__ a_out, int32_t* __restrict__ b_out) {
  const int64_t n = job.a_bins + job.b_bins;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (idx < job.a_bins && job.a_mode == kPairs) {
      const int64_t i = idx / E, j = idx - i * E;
      if (j < i) continue;
    }
    const int c = split_sum(partial + idx, n, job.splits);
    if (idx < job.a_bins)
      a_out[idx] = c;
    else
      b_out[idx - job.a_bins] = c;
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

int stats_check(int64_t T, int k, int E, const int32_t* topk, const int32_t* topk_next,
                int k_next, int E_next, const int32_t* expert_count, const int32_t* pair_count,
                const float* ochiai, const int32_t* transition) {
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
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_coact_stats_workspace_size(int64_t T, int E, int pairs, int E_next,
                                              size_t* ws_bytes) {
  if (ws_bytes == nullptr) return MOE_ERR_NULL;
  if (T < 0 || E < 1 || E > MOE_MAX_E || E_next < 0 || E_next > MOE_MAX_E) return MOE_ERR_SHAPE;
  *ws_bytes = moe::stats_workspace_bytes(moe::stats_job(T, E, pairs != 0, E_next > 0, E_next));
  return MOE_OK;
}

extern "C" int moe_coact_stats(const int32_t* topk, int64_t T, int k, int E,
                               const int32_t* topk_next, int k_next, int E_next,
                               int32_t* expert_count, int32_t* pair_count, float* ochiai,
                               int32_t* transition, int32_t* d_err, void* ws, size_t ws_bytes,
                               void* stream) {
  const int st = moe::stats_check(T, k, E, topk, topk_next, k_next, E_next, expert_count,
                                  pair_count, ochiai, transition);
  if (st != MOE_OK) return st;
  const moe::StatsJob job =
      moe::stats_job(T, E, pair_count != nullptr, transition != nullptr, E_next);
  if (ws == nullptr) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return MOE_ERR_ALIGN;
  if (ws_bytes < moe::stats_workspace_bytes(job)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);
  int32_t* partial = static_cast<int32_t*>(ws);
  // count (every partial bin of every split is written, also for T = 0)
  moe::stats_count_kernel<<<dim3(job.splits, job.a_slices + job.b_slices), moe::kStatThreads, 0,
                            s>>>(topk, Ti, k, E, topk_next, k_next, E_next, job, partial, d_err);
  MOE_CHECK_LAUNCH();
  moe::stats_sum_kernel<<<moe::grid_for(job.a_bins + job.b_bins), 256, 0, s>>>(
      partial, job, E, pair_count != nullptr ? pair_count : expert_count, transition);
  MOE_CHECK_LAUNCH();
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
