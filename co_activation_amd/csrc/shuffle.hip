// Token shuffle prediction.
//
// "Expert Coupling in MoE Pretraining ..." (abstract): token shuffling moves
// each token to the GPU predicted to hold its next-layer experts; the experts
// a token picks at one layer predict those it picks at the next.
//
//   M[i][r]     = sum_{j : p'(j) = r} X[i][j]       (64-bit, one block per i)
//   score_t[r]  = sum_{i in D_t} M[i][r],  pred_t = argmax_r, lowest r on ties
//
// The new token order is a stable counting sort by pred.  That sort is the
// dispatch plan with one source rank, one "expert" per token (its predicted
// rank) and the identity placement, so it reuses the plan kernels: the plan's
// row of token t is its new position and row_token is the inverse
// permutation.
#include "plan.hpp"

namespace moe {
namespace {

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct ShuffleWs {
  int64_t* M;
  int32_t* identity;
  int32_t* src1;
  int32_t* send_counts;
  int32_t* send_offsets;
  int64_t* counters;
  int32_t* perm_scratch;
  void* plan_ws;
  size_t bytes;
};

ShuffleWs shuffle_layout(void* base, int64_t T, int E, int G) {
  ShuffleWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  w.M = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * E * G));
  w.identity = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * G));
  w.src1 = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (G + 1)));
  w.send_counts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * G * G));
  w.send_offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (G * G + 1)));
  w.counters = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * 8));
  w.perm_scratch = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (T > 0 ? T : 1)));
  w.plan_ws = take(plan_workspace_bytes(T, G));
  w.bytes = off;
  return w;
}

constexpr int kScoreThreads = 256;

// One block per expert i of this layer: thread j adds X[i][j] into the sum of
// the rank that holds next-layer expert j (64-bit LDS atomics, exact), then
// thread r writes M[i][r].  Block 0 also writes the identity placement and
// the one-source offsets [0, T, ..., T] used by the sort.
__global__ __launch_bounds__(kScoreThreads) void rank_score_kernel(
    const int32_t* __restrict__ X, int E_next, const int32_t* __restrict__ expert_rank_next, int G,
    int T, int64_t* __restrict__ M, int32_t* __restrict__ identity, int32_t* __restrict__ src1,
    int32_t* d_err) {
  __shared__ unsigned long long sums[MOE_MAX_G];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < MOE_MAX_G) sums[tid] = 0;
  __syncthreads();
  int bad = 0;
  for (int j = tid; j < E_next; j += kScoreThreads) {
    const int r = expert_rank_next[j];
    if (r < 0 || r >= G) {
      bad = 1;
      continue;
    }
    const long long v = X[static_cast<int64_t>(i) * E_next + j];
    atomicAdd(&sums[r], static_cast<unsigned long long>(v));
  }
  __syncthreads();
  if (tid < G) M[static_cast<int64_t>(i) * G + tid] = static_cast<int64_t>(sums[tid]);
  if (i == 0) {
    if (bad) report(d_err, MOE_DERR_RANK_RANGE);
    if (tid < G) {
      identity[tid] = tid;
      src1[tid] = tid == 0 ? 0 : T;
    }
    if (tid == 0) src1[G] = T;
  }
}

// The prediction and the sort's first plan kernel in one pass.  Each block
// takes one 256-token tile: per token the k*G score sums and the argmax
// (ties to the lower rank; an all-zero score gives rank 0), written to
// pred_rank, the sort's one-slot routing; then the tile's count per rank
// from wave ballots, stored where the plan's count kernel stores them, with
// zero counter partials.  The sort continues with the plan's scan and write.
__global__ __launch_bounds__(kPlanTile) void predict_count_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int64_t* __restrict__ M, int G,
    int32_t* __restrict__ pred_rank, int32_t* __restrict__ tile_cnt, int64_t stride,
    int32_t* __restrict__ tile_stats, int32_t* d_err) {
  __shared__ int s_cnt[kPlanTile / kWave][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  const int t = blockIdx.x * kPlanTile + threadIdx.x;
  int best_r = -1;
  int errbits = 0;
  if (t < T) {
    int e[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      e[j] = -1;
      if (j < k) {
        const int v = topk[static_cast<int64_t>(t) * k + j];
        if (v >= 0 && v < E)
          e[j] = v;
        else
          errbits |= MOE_DERR_EXPERT_RANGE;
      }
    }
    long long best = 0;
    for (int r = 0; r < G; ++r) {
      long long sc = 0;
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (e[j] >= 0) sc += M[static_cast<int64_t>(e[j]) * G + r];
      if (r == 0 || sc > best) {
        best = sc;
        best_r = r;
      }
    }
    pred_rank[t] = best_r;
  }
  report(d_err, errbits);
  int mine = 0;
  for (int r = 0; r < G; ++r) {
    const uint64_t b = ballot(best_r == r);
    if (lane == r) mine = __popcll(b);
  }
  if (lane < G) s_cnt[wave][lane] = mine;
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(G)) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPlanTile / kWave; ++w) c += s_cnt[w][threadIdx.x];
    tile_cnt[static_cast<int64_t>(threadIdx.x) * stride + blockIdx.x] = c;
  }
  if (threadIdx.x < 4) tile_stats[static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x] = 0;
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Capacity-balanced shuffle: every rank receives exactly C = T/G tokens.
// Tokens in order take their best-scoring rank that still has room.  With
// the index f_r of the token that fills rank r (its C-th taker), token t's
// choice is its best rank with f_r >= t, independently of the other tokens;
// so the fill indices are found as a fixed point: start from "never full",
// assign every token, set f_r to the index of r's C-th taker, repeat.  The
// rank that fills first is exact after one round, the next after two, and
// so on: at most G rounds, stopping early once the f_r stop changing.

constexpr int kBalTile = 256;

// scores[t][r] = sum_{i in D_t} M[i][r]; block 0 also resets the
// convergence flag.
__global__ __launch_bounds__(kBalTile) void balanced_scores_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int64_t* __restrict__ M, int G,
    int64_t* __restrict__ scores, int32_t* __restrict__ flag, int32_t* d_err) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0;
  const int t = blockIdx.x * kBalTile + threadIdx.x;
  if (t >= T) return;
  int e[MOE_MAX_K];
  int errbits = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    e[j] = -1;
    if (j < k) {
      const int v = topk[static_cast<int64_t>(t) * k + j];
      if (v >= 0 && v < E)
        e[j] = v;
      else
        errbits |= MOE_DERR_EXPERT_RANGE;
    }
  }
  for (int r = 0; r < G; ++r) {
    long long sc = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j)
      if (e[j] >= 0) sc += M[static_cast<int64_t>(e[j]) * G + r];
    scores[static_cast<int64_t>(t) * G + r] = sc;
  }
  report(d_err, errbits);
}

constexpr int kBalWaves = kBalTile / kWave;
constexpr int kScorePre = 8;  // ranks whose scores a round kernel loads up front

// The fill index of every rank under one round's choices, into fill[] (LDS):
// for rank r, the tile where the running count of r's takers reaches cap,
// then the need-th taker inside that tile from the tile's taker masks (one
// 64-bit ballot per wave); "never full" when r has fewer than cap takers.
// The waves of the block take the ranks in turn.
__device__ void balanced_fill(const int32_t* __restrict__ tile_cnt,
                              const uint64_t* __restrict__ tile_mask, int NT, int G, int cap,
                              int* fill) {
  // A wave takes kGroup ranks at a time; their first kPre chunks of 64 tile
  // counts are loaded together before any is scanned.
  constexpr int kGroup = 2;
  constexpr int kPre = 4;
  const int lane = lane_id();
  const int wave = wave_id();
  for (int r0 = wave; r0 < G; r0 += kBalWaves * kGroup) {
    int pre[kGroup][kPre];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int r = r0 + g * kBalWaves;
#pragma unroll
      for (int c = 0; c < kPre; ++c) {
        const int j = c * kWave + lane;
        pre[g][c] = (r < G && j < NT) ? tile_cnt[static_cast<int64_t>(j) * G + r] : 0;
      }
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int r = r0 + g * kBalWaves;  // uniform across the wave
      if (r >= G) break;
      int carry = 0, hit = -1, need = 0;
      for (int base = 0, c = 0; base < NT && hit < 0; base += kWave, ++c) {
        const int j = base + lane;
        int v = 0;
        if (c < kPre) {
#pragma unroll
          for (int q = 0; q < kPre; ++q)
            if (q == c) v = pre[g][q];
        } else if (j < NT) {
          v = tile_cnt[static_cast<int64_t>(j) * G + r];
        }
        const int incl = wave_incl_scan(v) + carry;
        const uint64_t b = ballot(j < NT && incl >= cap);
        if (b) {
          const int first = __ffsll(static_cast<long long>(b)) - 1;
          hit = base + first;
          need = cap - (__shfl(incl, first, kWave) - __shfl(v, first, kWave));
        }
        carry = __shfl(incl, kWave - 1, kWave);
      }
      int nf = INT32_MAX;
      if (hit >= 0) {
        const uint64_t* m = tile_mask + (static_cast<int64_t>(hit) * G + r) * kBalWaves;
        uint64_t words[kBalWaves];
#pragma unroll
        for (int w = 0; w < kBalWaves; ++w) words[w] = m[w];
        int seen = 0;
#pragma unroll
        for (int w = 0; w < kBalWaves; ++w) {
          uint64_t bits = words[w];
          const int cnt = __popcll(bits);
          if (nf == INT32_MAX && seen + cnt >= need) {
            for (int q = 1; q < need - seen; ++q) bits &= bits - 1;
            nf = hit * kBalTile + w * kWave + (__ffsll(static_cast<long long>(bits)) - 1);
          }
          seen += cnt;
        }
      }
      if (lane == 0) fill[r] = nf;
    }
  }
}

// One round, one launch.  Every block first finds this round's fill indices
// from the previous round's per-tile counts and taker masks (the same in
// every block, so no block waits for another); if they equal the previous
// round's, the previous choices (in pred) are the fixed point and the round
// does nothing.  Otherwise every token takes its best rank with a fill index
// >= t, stored in pred, and the tile's counts and taker masks go to this
// round's half of the double buffers.  From round 2 on, tiles that end
// before the smallest fill index are skipped: those tokens choose freely in
// every round, and both halves already hold their counts and masks.
__global__ __launch_bounds__(kBalTile) void balanced_round_kernel(
    const int64_t* __restrict__ scores, int T, int G, int cap, int NT, int round,
    int32_t* __restrict__ tile_cnt, uint64_t* __restrict__ tile_mask,
    int32_t* __restrict__ fill_hist, int32_t* __restrict__ flag, int32_t* __restrict__ pred) {
  __shared__ int fill[MOE_MAX_G];
  __shared__ int s_cnt[kBalWaves][kWave];
  __shared__ int s_diff;
  if (round > 0 && *flag) return;
  const int cur = round & 1, prev = cur ^ 1;
  const int64_t half = static_cast<int64_t>(NT) * G;
  const int t = blockIdx.x * kBalTile + threadIdx.x;
  // Loads that do not depend on this round's fill indices go first, so their
  // latency overlaps the fill computation: the token's scores (up to
  // kScorePre ranks) and the previous round's fill index of rank threadIdx.x.
  long long sc[kScorePre];
#pragma unroll
  for (int r = 0; r < kScorePre; ++r)
    sc[r] = (t < T && r < G) ? scores[static_cast<int64_t>(t) * G + r] : 0;
  const int old_fill = (round > 0 && threadIdx.x < static_cast<unsigned>(G))
                           ? fill_hist[prev * G + threadIdx.x] : 0;
  if (threadIdx.x == 0) s_diff = 0;
  if (round == 0) {
    if (threadIdx.x < static_cast<unsigned>(G)) fill[threadIdx.x] = INT32_MAX;
  } else {
    balanced_fill(tile_cnt + prev * half, tile_mask + prev * half * kBalWaves, NT, G, cap, fill);
  }
  __syncthreads();
  if (round > 0) {
    if (threadIdx.x < static_cast<unsigned>(G) && fill[threadIdx.x] != old_fill) s_diff = 1;
    __syncthreads();
    if (!s_diff) {
      if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 1;
      return;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < static_cast<unsigned>(G))
    fill_hist[cur * G + threadIdx.x] = fill[threadIdx.x];
  if (round >= 2) {
    int min_fill = INT32_MAX;
    for (int r = 0; r < G; ++r) min_fill = min(min_fill, fill[r]);
    if (min_fill != INT32_MAX && (blockIdx.x + 1) * kBalTile <= min_fill) return;
  }
  const int lane = lane_id();
  const int wave = wave_id();
  // best rank with a fill index >= t: score descending, lower rank on ties
  int a = -1;
  if (t < T) {
    long long bs = 0;
    for (int r = 0; r < G; ++r) {
      if (fill[r] < t) continue;
      long long v = 0;
#pragma unroll
      for (int q = 0; q < kScorePre; ++q)
        if (q == r) v = sc[q];
      if (r >= kScorePre) v = scores[static_cast<int64_t>(t) * G + r];
      if (a < 0 || v > bs) {
        a = r;
        bs = v;
      }
    }
    pred[t] = a < 0 ? 0 : a;
  }
  uint64_t* mask = tile_mask + (cur * half + static_cast<int64_t>(blockIdx.x) * G) * kBalWaves;
  int mine = 0;
  for (int r = 0; r < G; ++r) {
    const uint64_t b = ballot(a == r);
    if (lane == r) {
      mine = __popcll(b);
      mask[static_cast<int64_t>(r) * kBalWaves + wave] = b;
    }
  }
  if (lane < G) s_cnt[wave][lane] = mine;
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(G)) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kBalWaves; ++w) c += s_cnt[w][threadIdx.x];
    tile_cnt[cur * half + static_cast<int64_t>(blockIdx.x) * G + threadIdx.x] = c;
  }
}

struct BalancedWs {
  ShuffleWs base;
  int64_t* scores;
  int32_t* fill_hist;  // [2][G]: the fill indices of the last two rounds
  int32_t* flag;
  int32_t* tile_cnt;   // [2][NT][G]
  uint64_t* tile_mask; // [2][NT][G][waves per tile]
  size_t bytes;
};

BalancedWs balanced_layout(void* base, int64_t T, int E, int G) {
  BalancedWs w{};
  w.base = shuffle_layout(base, T, E, G);
  char* p = static_cast<char*>(base);
  size_t off = w.base.bytes;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  const int64_t nt = (T + kBalTile - 1) / kBalTile;
  const int64_t ntc = nt > 0 ? nt : 1;
  w.scores = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * (T > 0 ? T : 1) * G));
  w.fill_hist = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 2 * G));
  w.flag = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  w.tile_cnt = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 2 * ntc * G));
  w.tile_mask = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * 2 * ntc * G * kBalWaves));
  w.bytes = off;
  return w;
}

}  // namespace
}  // namespace moe

extern "C" int moe_shuffle_balanced_workspace_size(int64_t T, int E, int G, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return MOE_ERR_NULL;
  if (T < 0 || E < 1 || E > MOE_MAX_E || G < 1 || G > MOE_MAX_G) return MOE_ERR_SHAPE;
  *ws_bytes = moe::balanced_layout(nullptr, T, E, G).bytes;
  return MOE_OK;
}

extern "C" int moe_shuffle_balanced(const int32_t* topk, int64_t T, int k, int E,
                                    const int32_t* transition, int E_next,
                                    const int32_t* expert_rank_next, int G, int32_t* pred_rank,
                                    int32_t* dest_pos, int32_t* perm, int32_t* shard_offsets,
                                    int32_t* d_err, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_E || E_next < 1 ||
      E_next > MOE_MAX_E || G < 1 || G > MOE_MAX_G ||
      T * static_cast<int64_t>(k) >= (int64_t{1} << 31) || T % G != 0)
    return MOE_ERR_SHAPE;
  if (transition == nullptr || expert_rank_next == nullptr || shard_offsets == nullptr ||
      ws == nullptr)
    return MOE_ERR_NULL;
  if (T > 0 && (topk == nullptr || pred_rank == nullptr || dest_pos == nullptr))
    return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOE_ERR_ALIGN;
  const moe::BalancedWs w = moe::balanced_layout(ws, T, E, G);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);
  const int NT = static_cast<int>((T + moe::kBalTile - 1) / moe::kBalTile);
  const int blocks = NT > 0 ? NT : 1;

  moe::rank_score_kernel<<<E, moe::kScoreThreads, 0, s>>>(transition, E_next, expert_rank_next, G,
                                                          Ti, w.base.M, w.base.identity,
                                                          w.base.src1, d_err);
  MOE_CHECK_LAUNCH();
  moe::balanced_scores_kernel<<<blocks, moe::kBalTile, 0, s>>>(topk, Ti, k, E, w.base.M, G,
                                                               w.scores, w.flag, d_err);
  MOE_CHECK_LAUNCH();
  if (Ti > 0) {
    // Round i's fill indices have the first i ranks to fill exact, so round
    // G assigns with the fixed point (rounds stop early once it is seen).
    for (int round = 0; round <= G; ++round) {
      moe::balanced_round_kernel<<<NT, moe::kBalTile, 0, s>>>(
          w.scores, Ti, G, Ti / G, NT, round, w.tile_cnt, w.tile_mask, w.fill_hist, w.flag,
          pred_rank);
      MOE_CHECK_LAUNCH();
    }
  }
  moe::PlanArgs a{pred_rank,      nullptr,        Ti,        1,
                  G,              w.base.identity, G,        G,
                  w.base.src1,    T,              w.base.send_counts, w.base.send_offsets,
                  perm ? perm : w.base.perm_scratch, nullptr, dest_pos,
                  nullptr,        w.base.counters, d_err,    w.base.plan_ws,
                  shard_offsets};
  return moe::launch_plan(a, s);
}

extern "C" int moe_shuffle_predict_workspace_size(int64_t T, int E, int G, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return MOE_ERR_NULL;
  if (T < 0 || E < 1 || E > MOE_MAX_E || G < 1 || G > MOE_MAX_G) return MOE_ERR_SHAPE;
  *ws_bytes = moe::shuffle_layout(nullptr, T, E, G).bytes;
  return MOE_OK;
}

extern "C" int moe_shuffle_predict(const int32_t* topk, int64_t T, int k, int E,
                                   const int32_t* transition, int E_next,
                                   const int32_t* expert_rank_next, int G, int32_t* pred_rank,
                                   int32_t* dest_pos, int32_t* perm, int32_t* shard_offsets,
                                   int32_t* d_err, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_E || E_next < 1 ||
      E_next > MOE_MAX_E || G < 1 || G > MOE_MAX_G ||
      T * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (transition == nullptr || expert_rank_next == nullptr || shard_offsets == nullptr ||
      ws == nullptr)
    return MOE_ERR_NULL;
  if (T > 0 && (topk == nullptr || pred_rank == nullptr || dest_pos == nullptr))
    return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOE_ERR_ALIGN;
  const moe::ShuffleWs w = moe::shuffle_layout(ws, T, E, G);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);

  moe::rank_score_kernel<<<E, moe::kScoreThreads, 0, s>>>(transition, E_next, expert_rank_next, G, Ti,
                                                  w.M, w.identity, w.src1, d_err);
  MOE_CHECK_LAUNCH();
  // the sort's tiles: one source rank, 256 tokens each, numbered from 0
  const moe::PlanTiles tiles = moe::plan_tiles(w.plan_ws, T, G);
  if (Ti > 0) {
    moe::predict_count_kernel<<<(Ti + moe::kPlanTile - 1) / moe::kPlanTile, moe::kPlanTile, 0,
                                s>>>(topk, Ti, k, E, w.M, G, pred_rank, tiles.cnt, tiles.stride,
                                     tiles.stats, d_err);
    MOE_CHECK_LAUNCH();
  }
  moe::PlanArgs a{pred_rank,      nullptr,        Ti,        1,
                  G,              w.identity,     G,         G,
                  w.src1,         T,              w.send_counts, w.send_offsets,
                  perm ? perm : w.perm_scratch,   nullptr,   dest_pos,
                  nullptr,        w.counters,     d_err,     w.plan_ws,
                  shard_offsets};
  a.counts_ready = true;
  return moe::launch_plan(a, s);
}
