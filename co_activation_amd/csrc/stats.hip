// Co-activation statistics of one MoE layer.
//
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training" (Key Observation): the set of tokens that activate each expert
// and the Ochiai similarity |A n B| / sqrt(|A| |B|) of two experts.
// "Expert Coupling in MoE Pretraining ..." (abstract): expert pairs selected
// together in a layer, and the experts of one layer predicting those of the
// next (transition counts).
//
// Three kernels, no global atomics:
//   count  : the tokens are cut into splits and the counted matrices into
//            slices of whole rows; block (split, slice) counts its split's
//            tokens into an LDS histogram of its slice (16-bit counters, two
//            per word, while a split has fewer than 2^16 tokens) and copies
//            the histogram to its own region of the workspace.  The pair
//            matrix is counted on and above the diagonal only, its rows
//            packed (row i holds columns i..E-1): a token adds one to (i, j)
//            for each of its experts i inside the slice's rows and each of
//            its experts j >= i.
//   sum    : one block per output row; the splits' partials of each bin are
//            added in a fixed order (integer addition, so the counts do not
//            depend on scheduling).
//   finish : mirrors the pair matrix, copies the diagonal out as the
//            per-expert counts and evaluates Ochiai in double precision.
// Every output element is written, so nothing needs clearing first.
#include "common.hpp"

namespace moe {
namespace {

// Four-wave blocks, like the combine's: the statistics of one batch run on a
// second stream beside the previous batch's combine, and a block has to find
// room on a CU that the combine keeps busy.  Eight-wave blocks count a little
// faster alone (workload 5: 15.9 against 18.9 us) but wait for whole CUs to
// drain, which made the two-batch pipelined step 0.612 -> 0.671 ms.
constexpr int kStatThreads = 256;
// Tokens per split, one per thread, until kMaxSplits: more, smaller splits
// keep every CU counting (512-token splits took 11.4 us to count at T = 32768,
// E = 256, k = 8, these 8.2) at the price of twice the partials to sum.
constexpr int kSplitTokens = 256;
constexpr int kMaxSplits = 128;
constexpr int kSliceBytes = 32768;  // LDS histogram of one block
constexpr int kMaxSlices = 16;      // at most 5 + 8 for E = E_next = 256

enum StatMode { kCounts = 0, kPairs = 1, kTransitions = 2 };

// First bin of packed row i of an E x E upper triangle.
__host__ __device__ __forceinline__ int tri_row(int i, int E) { return i * E - (i * (i - 1)) / 2; }

// Work of one statistics call.  Matrix A is the per-expert counts (E bins,
// one slice) or the packed pair triangle (E (E + 1) / 2 bins); matrix B the
// transitions (E x E_next bins).  Slices [0, a_slices) cover rows of A, the
// rest rows of B: slice q holds rows [r0[q], r1[q]) starting at bin bin0[q]
// of its matrix and at word w0[q] of a split's partial row (row_words words;
// a 32-bit word holds two 16-bit bins, or one 32-bit bin when wide).
struct StatsJob {
  int a_mode;  // kCounts or kPairs
  int E, E_next;
  int a_slices, b_slices;
  int wide;
  int splits, split_tokens;
  int64_t row_words;
  int r0[kMaxSlices], r1[kMaxSlices], bin0[kMaxSlices], w0[kMaxSlices];
};

StatsJob stats_job(int64_t T, int E, bool pairs, bool transitions, int E_next) {
  StatsJob j{};
  j.a_mode = pairs ? kPairs : kCounts;
  j.E = E;
  j.E_next = transitions ? E_next : 0;
  int64_t splits = (T + kSplitTokens - 1) / kSplitTokens;
  if (splits < 1) splits = 1;
  if (splits > kMaxSplits) splits = kMaxSplits;
  j.splits = static_cast<int>(splits);
  j.split_tokens = static_cast<int>((T + splits - 1) / splits);
  j.wide = j.split_tokens > 65535;
  const int cap = (kSliceBytes / 4) * (j.wide ? 1 : 2);  // bins per slice
  int n = 0;
  int64_t w = 0;
  auto add = [&](int r0, int r1, int b0, int nb) {
    j.r0[n] = r0;
    j.r1[n] = r1;
    j.bin0[n] = b0;
    j.w0[n] = static_cast<int>(w);
    w += j.wide ? nb : (nb + 1) / 2;
    w = (w + 3) & ~int64_t{3};  // 16-byte aligned slice regions
    ++n;
  };
  if (!pairs) {
    add(0, E, 0, E);
  } else {
    for (int r = 0; r < E;) {
      int r1 = r, nb = 0;
      while (r1 < E && nb + (E - r1) <= cap) nb += E - r1++;
      add(r, r1, tri_row(r, E), nb);
      r = r1;
    }
  }
  j.a_slices = n;
  if (transitions) {
    const int per = cap / E_next;
    for (int r = 0; r < E; r += per) {
      const int r1 = r + per < E ? r + per : E;
      add(r, r1, r * E_next, (r1 - r) * E_next);
    }
  }
  j.b_slices = n - j.a_slices;
  // Split stride: an odd number of 256-byte units, so that the copies of a
  // bin in the splits' rows do not all fall on the same memory channels
  // (a stride near a multiple of 64 KB made the sum several times slower).
  w = (w + 63) & ~int64_t{63};
  if (((w / 64) & 1) == 0) w += 64;
  j.row_words = w;
  return j;
}

size_t stats_workspace_bytes(const StatsJob& j) {
  const size_t b = sizeof(uint32_t) * static_cast<size_t>(j.splits) * j.row_words;
  return (b + 255) & ~static_cast<size_t>(255);
}

// Reads one token's ids into e[]; an out-of-range slot, and a slot that
// repeats an earlier one, become -1 (so a token adds at most one to a bin).
__device__ __forceinline__ int load_ids(const int32_t* __restrict__ row, int k, int E,
                                        int (&e)[MOE_MAX_K]) {
  int err = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    e[j] = -1;
    if (j < k) {
      const int v = row[j];
      bool dup = false;
#pragma unroll
      for (int q = 0; q < j; ++q) dup |= e[q] == v;
      if (v < 0 || v >= E)
        err |= MOE_DERR_EXPERT_RANGE;
      else if (dup)
        err |= MOE_DERR_EXPERT_DUP;
      else
        e[j] = v;
    }
  }
  return err;
}

// Adds one to local bin b of the slice.
template <bool WIDE>
__device__ __forceinline__ void bump(unsigned* hist, int b) {
  if constexpr (WIDE)
    atomicAdd(&hist[b], 1u);
  else
    atomicAdd(&hist[b >> 1], 1u << ((b & 1) * 16));
}

template <bool WIDE>
__global__ __launch_bounds__(kStatThreads) void stats_count_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int32_t* __restrict__ topk2,
    int k2, int E2, StatsJob job, uint32_t* __restrict__ partial, int32_t* d_err) {
  __shared__ __align__(16) unsigned hist[kSliceBytes / 4];
  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const bool in_a = q < job.a_slices;
  const int mode = in_a ? job.a_mode : kTransitions;
  const int r0 = job.r0[q], r1 = job.r1[q], bin0 = job.bin0[q];
  const int nb = mode == kPairs ? tri_row(r1, E) - bin0 : (mode == kCounts ? E : (r1 - r0) * E2);
  const int vecs = ((WIDE ? nb : (nb + 1) / 2) + 3) / 4;  // 16-byte vectors of the slice
  uint4* hv = reinterpret_cast<uint4*>(hist);
  for (int i = threadIdx.x; i < vecs; i += kStatThreads) hv[i] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  const int tb0 = split * job.split_tokens;
  const int tb1 = min(T, tb0 + job.split_tokens);
  int errbits = 0;
  for (int t = tb0 + static_cast<int>(threadIdx.x); t < tb1; t += kStatThreads) {
    int e[MOE_MAX_K];
    errbits |= load_ids(topk + static_cast<int64_t>(t) * k, k, E, e);
    if (mode == kCounts) {
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a)
        if (e[a] >= 0) bump<WIDE>(hist, e[a]);
    } else if (mode == kPairs) {
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a) {
        const int i = e[a];
        if (i < r0 || i >= r1) continue;
        const int base = tri_row(i, E) - i - bin0;
#pragma unroll
        for (int b = 0; b < MOE_MAX_K; ++b)
          if (e[b] >= i) bump<WIDE>(hist, base + e[b]);
      }
    } else {
      int f[MOE_MAX_K];
      errbits |= load_ids(topk2 + static_cast<int64_t>(t) * k2, k2, E2, f);
#pragma unroll
      for (int a = 0; a < MOE_MAX_K; ++a) {
        const int i = e[a];
        if (i < r0 || i >= r1) continue;
        const int base = (i - r0) * E2;
#pragma unroll
        for (int b = 0; b < MOE_MAX_K; ++b)
          if (f[b] >= 0) bump<WIDE>(hist, base + f[b]);
      }
    }
  }
  // One slice of each matrix reports the data errors it saw.
  if (q == 0 || q == job.a_slices) report(d_err, errbits);
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(partial + static_cast<int64_t>(split) * job.row_words +
                                        job.w0[q]);
  for (int i = threadIdx.x; i < vecs; i += kStatThreads) dst[i] = hv[i];
}

// One block per output row: the pair matrix's rows (columns j >= i; the
// finish kernel fills the rest) or the single row of per-expert counts,
// then the transition rows.  The splits' partials of a bin are added with
// sixteen independent loads in flight (eight left the latency exposed,
// thirty-two slowed the memory side).
template <bool WIDE>
__global__ void stats_sum_kernel(const uint32_t* __restrict__ partial, StatsJob job,
                                 int32_t* __restrict__ a_out, int32_t* __restrict__ b_out) {
  const int E = job.E;
  const int a_rows = job.a_mode == kPairs ? E : 1;
  int row = blockIdx.x;
  const bool in_a = row < a_rows;
  if (!in_a) row -= a_rows;
  const int cols = in_a ? E : job.E_next;
  int q = in_a ? 0 : job.a_slices;
  const int q_end = in_a ? job.a_slices : job.a_slices + job.b_slices;
  while (q + 1 < q_end && job.r0[q + 1] <= row) ++q;
  const uint32_t* p = partial + job.w0[q];
  for (int j = threadIdx.x; j < cols; j += blockDim.x) {
    int b;  // bin inside the slice
    if (!in_a)
      b = (row - job.r0[q]) * job.E_next + j;
    else if (job.a_mode == kCounts)
      b = j;
    else if (j >= row)
      b = tri_row(row, E) - job.bin0[q] + (j - row);
    else
      continue;
    const int64_t word = WIDE ? b : (b >> 1);
    const int sh = WIDE ? 0 : (b & 1) * 16;
    const uint32_t mask = WIDE ? 0xFFFFFFFFu : 0xFFFFu;
    constexpr int kLoads = 16;
    uint32_t acc[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc[u] = 0u;
    int sp = 0;
    for (; sp + kLoads <= job.splits; sp += kLoads) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) acc[u] += (p[(sp + u) * job.row_words + word] >> sh) & mask;
    }
    for (; sp < job.splits; ++sp) acc[0] += (p[sp * job.row_words + word] >> sh) & mask;
    uint32_t total = 0u;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) total += acc[u];
    const int c = static_cast<int>(total);
    if (!in_a)
      b_out[static_cast<int64_t>(row) * job.E_next + j] = c;
    else if (job.a_mode == kCounts)
      a_out[j] = c;
    else
      a_out[static_cast<int64_t>(row) * E + j] = c;
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
  uint32_t* partial = static_cast<uint32_t*>(ws);
  // count (every slice region of every split's partial row is written, also
  // for T = 0)
  const dim3 grid(job.splits, job.a_slices + job.b_slices);
  if (job.wide)
    moe::stats_count_kernel<true><<<grid, moe::kStatThreads, 0, s>>>(
        topk, Ti, k, E, topk_next, k_next, E_next, job, partial, d_err);
  else
    moe::stats_count_kernel<false><<<grid, moe::kStatThreads, 0, s>>>(
        topk, Ti, k, E, topk_next, k_next, E_next, job, partial, d_err);
  MOE_CHECK_LAUNCH();
  const unsigned rows = (pair_count != nullptr ? E : 1) + (transition != nullptr ? E : 0);
  int32_t* a_out = pair_count != nullptr ? pair_count : expert_count;
  if (job.wide)
    moe::stats_sum_kernel<true><<<rows, 256, 0, s>>>(partial, job, a_out, transition);
  else
    moe::stats_sum_kernel<false><<<rows, 256, 0, s>>>(partial, job, a_out, transition);
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
