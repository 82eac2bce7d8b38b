// Token shuffle prediction.
//
// "Expert Coupling in MoE Pretraining ..." (abstract): tokens are reordered
// by the rank forecast for their next-layer experts, the forecast resting on
// how well one layer's expert choices anticipate the next layer's.
//
//   M[i][r]     = sum_{j : p'(j) = r} X[i][j]       (64-bit, one block per i)
//   score_t[r]  = sum_{i in D_t} M[i][r],  pred_t = argmax_r, lowest r on ties
//
// The new token order is a stable counting sort by pred.  That sort is the
// dispatch plan with one source rank, one "expert" per token (its predicted
// rank) and the identity placement, so it reuses the plan kernels: the plan's
// row of token t is its new position and row_token is the inverse
// permutation.
#include <climits>
#include <mutex>

#include "plan.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
  uint64_t* rec;  // exchange words of the exchange form: [kXSlots][kXBlocks][G + 1]
  size_t bytes;
};

constexpr int kXBlocksMax = 128;  // kXBlocks, needed before the kernels
constexpr int kXSlots = 4;        // rounds whose exchange words are kept at once

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
  w.rec = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * kXSlots * kXBlocksMax * (G + 1)));
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
          need = cap - (lane_value(incl, first) - lane_value(v, first));
        }
        carry = lane_value(incl, kWave - 1);
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

// ---------------------------------------------------------------------------
// Balanced shuffle in one launch (after the preference lists), for inputs
// whose tokens fit in at most kXBlocks blocks of kXThreads threads with up
// to kXMaxTpt tokens per thread, all resident at once (checked on the host);
// larger inputs take the round-per-launch kernels above.
//
// rank_argmax_kernel (the free shuffle's prediction above 16 ranks) and
// prefs_sort_kernel (the balanced shuffle's preference lists) read each
// token's rows of M with a group of lanes per token.
//
// shuffle_exchange_kernel: block b owns tokens [b * TB, (b + 1) * TB).  Each
// round every token takes its first preference r with t <= limit[r],
// limit[r] being the fill index of r under the previous round's choices (a
// choice stands while its rank still takes the token: the limits only move
// earlier from round to round); the
// block counts its tokens per (64-token chunk, rank) with LDS atomics and
// publishes its counts per rank as 64-bit words tagged with the round, in a
// ring of kXSlots rounds, with a flag saying whether any of its tokens
// changed its choice.  Every block reads the counts of the blocks before it
// for this round, and all blocks' flags of the previous round (not of this
// one, so that no block waits for a later, slower block's current round).
// That prefix and the block's own chunk counts give the next round's limits:
// a rank full before the block, open after it, or filled at an exact
// position inside it.  The rounds stop one round after the first in which no
// token of any block changed its choice (the fixed point, reached within
// G + 1 rounds; the extra round repeats it).  Every block has published the
// previous round before a block moves on, so a block writing round n + 1
// knows that all blocks have read round n - 3: four slots suffice.  The
// final counts then give each token its position directly:
// its rank's shard offset r * cap, plus the rank's tokens in earlier blocks,
// earlier chunks, and earlier lanes of its chunk -- the stable counting sort,
// without the plan kernels.
//
// The blocks wait on each other, so they must all be resident at once; next
// to a kernel that keeps the CUs busy (another stream) they wait for it to
// drain.  Waits poll the tagged words with agent-scope atomic loads; every
// poll loop gives up after a bound, reporting MOE_DERR_SYNC, so a block
// that waits for a block that never publishes still exits.

constexpr int kXThreads = 1024;
constexpr int kXWaves = kXThreads / kWave;
constexpr int kXBlocks = kXBlocksMax;
constexpr int kXMaxTpt = 4;
constexpr int kXChunks = kXMaxTpt * kXWaves;  // 64-token chunks per block
constexpr unsigned kXSpinLimit = 1u << 22;     // polls (about 1 us each) before giving up
constexpr int kXGroups = 16;  // thread groups that share out the earlier blocks' counts

inline int group_width(int G) {
  int w = 1;
  while (w < G) w <<= 1;
  return w;
}

// Preference rows are padded to 16 bytes so that each starts aligned.
inline int64_t pref_stride(int G) { return (G + 15) / 16 * 16; }

// Tokens per lane group (t0 + u, u < kScoreTokens): their id loads and then
// their row loads go out together.  One measured fastest (rows of M are read
// from L2, which more tokens in flight per wave do not speed up).
constexpr int kScoreTokens = 1;

// Scores of tokens t0 + u for rank r (lane r of the group): the sums of the
// tokens' rows of M (0 for tokens at or past T).
__device__ __forceinline__ void token_scores(const int32_t* __restrict__ topk, int t0, int T,
                                             int k, int E, const int64_t* __restrict__ M, int G,
                                             int r, long long (&score)[kScoreTokens],
                                             int& errbits) {
  int e[kScoreTokens][MOE_MAX_K];
#pragma unroll
  for (int u = 0; u < kScoreTokens; ++u) {
    const int t = t0 + u;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j)
      e[u][j] = (j < k && t < T) ? topk[static_cast<int64_t>(t) * k + j] : -1;
  }
  // every row load goes out before the first add
#pragma unroll
  for (int u = 0; u < kScoreTokens; ++u) {
    long long m[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      const int x = e[u][j];
      const bool ok = j < k && x >= 0 && x < E && r < G;
      m[j] = ok ? M[static_cast<int64_t>(x) * G + r] : 0;
      if (j < k && (x < 0 || x >= E) && t0 + u < T) errbits |= MOE_DERR_EXPERT_RANGE;
    }
    long long sc = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) sc += m[j];
    score[u] = sc;
  }
}

// The value of lane (lane ^ j), j a power of two below 64 that is a
// constant once the caller's loop is unrolled: DPP lane moves for j = 1, 2
// (quad permutes), 4 (row shifts) and 8 (row rotate), a swizzle inside 32
// lanes for j = 16, an LDS permute only for j = 32.
__device__ __forceinline__ int xor_lane(int v, int j) {
  switch (j) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
      return (lane_id() & 4) ? dn : up;
    }
    case 8: return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 16: return __builtin_amdgcn_ds_swizzle(v, 0x401F);  // and 0x1f, xor 0x10
    default: return __shfl_xor(v, j, kWave);
  }
}

__device__ __forceinline__ long long xor_lane(long long v, int j) {
  const int lo = xor_lane(static_cast<int>(static_cast<unsigned long long>(v)), j);
  const int hi = xor_lane(static_cast<int>(static_cast<unsigned long long>(v) >> 32), j);
  return static_cast<long long>((static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
                                static_cast<uint32_t>(lo));
}

// Scores below 2^25 (scores are counts, never negative) make keys
// score * 64 + (63 - r) below 2^31 that order exactly as the 64-bit ones; a
// wave takes the 32-bit form when all its lanes' scores allow it.
constexpr long long kKey32Limit = 1ll << 25;

// The free shuffle's prediction: a group of W lanes (W = G rounded up to a
// power of two) per token; lane r adds the token's rows of M for rank r
// (coalesced across the group), and a max-reduction over the keys
// score * 64 + (63 - r) (ties to the lower rank) gives the first rank.
// Also clears the exchange words.
template <int W>
__global__ __launch_bounds__(256) void rank_argmax_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int64_t* __restrict__ M, int G,
    int32_t* __restrict__ pred, uint64_t* __restrict__ rec, int64_t rec_words, int32_t* d_err) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < rec_words; i += gridDim.x * 256ll) rec[i] = 0;
  const int per_block = 256 / W;
  const int tg = (blockIdx.x * per_block + static_cast<int>(threadIdx.x) / W) * kScoreTokens;
  const int r = static_cast<int>(threadIdx.x) % W;
  int errbits = 0;
  long long score[kScoreTokens];
  token_scores(topk, tg, T, k, E, M, G, r, score, errbits);
  if (r == 0) report(d_err, errbits);
#pragma unroll
  for (int u = 0; u < kScoreTokens; ++u) {
    const int t = tg + u;
    const bool live = t < T && r < G;
    bool top;
    if (ballot(score[u] >= kKey32Limit) == 0) {
      const int key = live ? static_cast<int>(score[u]) * 64 + (63 - r) : -1;
      int best = key;
#pragma unroll
      for (int d = 1; d < W; d <<= 1) best = max(best, xor_lane(best, d));
      top = key == best;
    } else {
      const long long key = live ? score[u] * 64 + (63 - r) : LLONG_MIN;
      long long best = key;
#pragma unroll
      for (int d = 1; d < W; d <<= 1) best = max(best, xor_lane(best, d));
      top = key == best;
    }
    if (live && top) pred[t] = r;
  }
}

// The balanced shuffle's preference lists: a group of W lanes per token as
// in rank_argmax_kernel, then a bitonic sort of the group's keys, descending,
// across its lanes (W log W compare-exchanges on the lanes' shuffled keys,
// against W^2 comparisons for ranking by counting) leaves the i-th preferred
// rank in lane i of the group, which writes it at byte pref_byte(i) of the
// token's row.  Also clears the exchange words.
//
// A row holds groups of 16 positions, each group transposed: its 32-bit
// word d holds positions d, d + 4, d + 8, d + 12 (byte j: position 4j + d),
// so that a test of all 16 positions a word at a time (first_feasible)
// yields its result bits in position order.
__host__ __device__ inline int pref_byte(int i) {
  return (i & ~15) | ((i & 3) << 2) | ((i >> 2) & 3);
}

template <int W, typename K>
__device__ __forceinline__ K bitonic_desc(K key, int r) {
#pragma unroll
  for (int size = 2; size <= W; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      const K other = xor_lane(key, j);
      const bool lower = (r & j) == 0;
      const bool desc = (r & size) == 0;
      key = (lower == desc) ? max(key, other) : min(key, other);
    }
  }
  return key;
}

template <int W>
__global__ __launch_bounds__(256) void prefs_sort_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int64_t* __restrict__ M, int G,
    int64_t Gs, uint8_t* __restrict__ prefs, uint64_t* __restrict__ rec, int64_t rec_words,
    int32_t* d_err) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < rec_words; i += gridDim.x * 256ll) rec[i] = 0;
  const int per_block = 256 / W;
  const int tg = (blockIdx.x * per_block + static_cast<int>(threadIdx.x) / W) * kScoreTokens;
  const int r = static_cast<int>(threadIdx.x) % W;
  int errbits = 0;
  long long score[kScoreTokens];
  token_scores(topk, tg, T, k, E, M, G, r, score, errbits);
  if (r == 0) report(d_err, errbits);
#pragma unroll
  for (int u = 0; u < kScoreTokens; ++u) {
    const int t = tg + u;
    const bool live = t < T && r < G;
    int rank;
    if (ballot(score[u] >= kKey32Limit) == 0) {
      const int key =
          bitonic_desc<W, int>(live ? static_cast<int>(score[u]) * 64 + (63 - r) : -1, r);
      rank = 63 - (key & 63);
    } else {
      const long long key =
          bitonic_desc<W, long long>(live ? score[u] * 64 + (63 - r) : LLONG_MIN, r);
      rank = 63 - static_cast<int>(key & 63);
    }
    if (live) prefs[static_cast<int64_t>(t) * Gs + pref_byte(r)] = static_cast<uint8_t>(rank);
  }
}

// One 64-bit exchange word: the round tag (round + 1) above the value.
__device__ __forceinline__ uint64_t xword(int round, uint32_t v) {
  return (static_cast<uint64_t>(round + 1) << 32) | v;
}

// Polls *w until it carries this round's tag; false after the spin bound.
__device__ __forceinline__ bool xwait(const uint64_t* w, int round, uint32_t& v) {
  const uint64_t want = static_cast<uint64_t>(round + 1);
  for (unsigned spin = 0; spin < kXSpinLimit; ++spin) {
    const uint64_t x = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((x >> 32) == want) {
      v = static_cast<uint32_t>(x);
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Sum of the words w[c * stride], w[(c + ng) * stride], ... for indices
// below n once each carries this round's tag: the loads go out four at a
// time, all four before the first wait.
__device__ __forceinline__ bool xsum(const uint64_t* w, int64_t stride, int c, int ng, int n,
                                     int round, int& sum) {
  const uint64_t want = static_cast<uint64_t>(round + 1);
  int acc = 0;
  for (int j0 = c; j0 < n; j0 += 4 * ng) {
    uint64_t x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q * ng;
      x[q] = j < n ? __hip_atomic_load(w + j * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q * ng;
      if (j < n) {
        uint32_t v = static_cast<uint32_t>(x[q]);
        if ((x[q] >> 32) != want && !xwait(w + j * stride, round, v)) return false;
        acc += static_cast<int>(v);
      }
    }
  }
  sum = acc;
  return true;
}

// The ranks in each group of 16 preferences.
template <int PW>
__device__ __forceinline__ void group_masks(const u32x4 (&pw)[PW], int G, uint64_t (&gm)[PW]) {
#pragma unroll
  for (int w = 0; w < PW; ++w) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // position w * 16 + i: word i & 3, byte i >> 2
      const uint32_t p = (pw[w][i & 3] >> (8 * (i >> 2))) & 0xFFu;
      if (w * 16 + i < G) m |= 1ull << p;
    }
    gm[w] = m;
  }
}

// The first rank at position >= start of the preference list pw that feas
// holds, and its position (the last preference, position G - 1, when none
// does).  gm holds the ranks of each group of 16 preferences: the group of
// the answer is the first one at or after start's whose ranks meet feas
// (ranks listed before start are infeasible), so that only that group's 16
// positions are tested, four at a time: the bit of feas for rank p is bit
// p & 7 of byte p >> 3, so one byte permute of feas fetches each position's
// byte, a second turns p & 7 into a one-hot byte, and a byte that keeps a
// bit after the AND sets its bit 7 in x + 0x7f (no carry leaves a byte).
template <int PW>
__device__ __forceinline__ int first_feasible(const u32x4 (&pw)[PW], const uint64_t (&gm)[PW],
                                              int G, uint64_t feas, int start, int& pos) {
  int gsel = -1;
#pragma unroll
  for (int w = PW - 1; w >= 0; --w)
    if (w * 16 < G && w * 16 + 16 > start && (gm[w] & feas) != 0) gsel = w;
  if (gsel >= 0) {
    uint32_t g[4] = {pw[0][0], pw[0][1], pw[0][2], pw[0][3]};
#pragma unroll
    for (int w = 1; w < PW; ++w) {
      const bool sel = w == gsel;
#pragma unroll
      for (int j = 0; j < 4; ++j) g[j] = sel ? pw[w][j] : g[j];
    }
    const uint32_t lo = static_cast<uint32_t>(feas), hi = static_cast<uint32_t>(feas >> 32);
    // bit 8j + d of m: position 4j + d of the group is feasible (bit order
    // is position order)
    uint32_t m = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t fb = __builtin_amdgcn_perm(hi, lo, (g[d] >> 3) & 0x07070707u);
      const uint32_t oh = __builtin_amdgcn_perm(0x80402010u, 0x08040201u, g[d] & 0x07070707u);
      m |= (((fb & oh) + 0x7F7F7F7Fu) & 0x80808080u) >> (7 - d);
    }
    const int n = G - gsel * 16;  // positions the group holds
    if (n < 16) m &= (1u << ((n >> 2) * 8 + (n & 3))) - 1u;
    const int s0 = start - gsel * 16;
    if (s0 > 0) m &= ~((1u << ((s0 >> 2) * 8 + (s0 & 3))) - 1u);
    if (m != 0) {
      const int b = __ffs(m) - 1;
      const int j = b >> 3, d = b & 7;
      pos = gsel * 16 + 4 * j + d;
      const uint32_t gd = d == 0 ? g[0] : d == 1 ? g[1] : d == 2 ? g[2] : g[3];
      return static_cast<int>((gd >> (8 * j)) & 0xFFu);
    }
  }
  const int i = (G - 1) & 15, w = (G - 1) >> 4;
  int last = 0;
#pragma unroll
  for (int q = 0; q < PW; ++q)
    if (q == w) last = static_cast<int>((pw[q][i & 3] >> (8 * (i >> 2))) & 0xFFu);
  pos = G - 1;
  return last;
}

template <int PW>
__global__ __launch_bounds__(kXThreads) void shuffle_exchange_kernel(
    const uint8_t* __restrict__ prefs, int64_t Gs, int T, int G, int cap, int TB, int tpt, int nb,
    uint64_t* __restrict__ rec, int32_t* __restrict__ pred_rank, int32_t* __restrict__ dest_pos,
    int32_t* __restrict__ perm, int32_t* __restrict__ shard_offsets, int32_t* d_err) {
  __shared__ uint8_t s_choice[kXMaxTpt * kXThreads];  // each token's current choice
  __shared__ uint8_t s_cursor[kXMaxTpt * kXThreads];  // its position in the token's list
  // Rank r takes tokens t <= s_lim[r] of this block: INT_MAX for a rank
  // still open after the block, -1 for one full before it, else the position
  // of its cap-th taker.
  __shared__ int s_lim[MOE_MAX_G];
  __shared__ int s_cc[kXChunks][MOE_MAX_G];  // tokens per (64-token chunk, rank)
  // This block's tokens per rank, kept by LDS atomics as tokens change
  // their choices; the earlier blocks' (the prefix), summed by LDS atomics
  // into the half of the round's parity, the other half, last read in the
  // previous round, cleared for the next one.
  __shared__ int s_cnt[MOE_MAX_G];
  __shared__ int s_pre[2][MOE_MAX_G];
  __shared__ int s_abort, s_changed;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = lane_id();
  const int wave = wave_id();
  const int b = blockIdx.x;
  const int t0 = b * TB;
  const int nchunks = tpt * kXWaves;
  const int64_t words = static_cast<int64_t>(G) + 1;  // per block and round: G counts, a flag
  constexpr int ng = kXGroups;  // thread (c, r), c < 16, r < G <= 64

  if (tid < MOE_MAX_G) {
    s_lim[tid] = INT_MAX;
    s_cnt[tid] = 0;
    s_pre[0][tid] = 0;
  }
  if (tid == 0) s_abort = 0;
  for (int u = 0; u < tpt; ++u) {
    s_choice[u * kXThreads + tid] = 255;
    s_cursor[u * kXThreads + tid] = 0;
  }
  __syncthreads();

  // A token's preferences and the ranks of each group of 16 of them; with
  // one token per thread they stay in registers for all rounds.
  //
  // The fill positions only move earlier from round to round (a rank that
  // closes earlier sends its later takers to their next choices, which fill
  // those ranks no later), so a rank a token once found full stays full: a
  // choice stands while it is feasible, and otherwise the search resumes
  // after it.
  u32x4 pw1[PW];
  uint64_t gm1[PW];
#pragma unroll
  for (int w = 0; w < PW; ++w) pw1[w] = u32x4{0u, 0u, 0u, 0u};
  if (tpt == 1 && t0 + tid < T) {
#pragma unroll
    for (int w = 0; w < PW; ++w)
      pw1[w] = *reinterpret_cast<const u32x4*>(prefs + static_cast<int64_t>(t0 + tid) * Gs + 16 * w);
  }
  group_masks<PW>(pw1, G, gm1);

  const int max_rounds = G + 3;
  int P = 0;  // lane r: tokens rank r took in earlier blocks (this round)
  int c1 = 255, cur1 = 0;  // with one token per thread: its choice and cursor
  for (int round = 0; round < max_rounds; ++round) {
    uint64_t* xr = rec + static_cast<int64_t>(round % kXSlots) * nb * words;
    const int par = round & 1;
    if (tid < MOE_MAX_G) s_pre[par ^ 1][tid] = 0;
    // 1. choices; a token that changes moves its counts (per chunk and rank,
    // per rank)
    int changed = round == 0 ? 1 : 0;
    for (int u = 0; u < tpt; ++u) {
      const int t = t0 + u * kXThreads + tid;
      const int idx = u * kXThreads + tid;
      int c = tpt == 1 ? c1 : s_choice[idx];
      const int c0 = c;
      // no choice yet, or its rank is full
      const bool walk = t < T && (c >= G || t > s_lim[c]);
      if (ballot(walk) != 0) {
        // The ranks feasible for the wave's tokens base .. base + 63: those
        // taking all of them, and those whose cap-th taker is among them
        // (feasible for the tokens up to it).
        const int base = t0 + u * kXThreads + wave * kWave;
        const int lim = lane < G ? s_lim[lane] : -1;
        uint64_t feas = ballot(lim >= base + kWave - 1);
        uint64_t part = ballot(lim >= base && lim < base + kWave - 1);
        while (part != 0) {
          const int r = __ffsll(static_cast<long long>(part)) - 1;
          part &= part - 1;
          if (__builtin_amdgcn_readlane(lim, r) >= t) feas |= 1ull << r;
        }
        if (walk) {
          if (tpt != 1) {  // several tokens per thread: this one's preferences
#pragma unroll
            for (int w = 0; w < PW; ++w)
              pw1[w] = *reinterpret_cast<const u32x4*>(prefs + static_cast<int64_t>(t) * Gs + 16 * w);
            group_masks<PW>(pw1, G, gm1);
          }
          const int start = c >= G ? 0 : (tpt == 1 ? cur1 : s_cursor[idx]) + 1;
          int pos = 0;
          const int nw = first_feasible<PW>(pw1, gm1, G, feas, start, pos);
          s_cursor[idx] = static_cast<uint8_t>(pos);
          cur1 = pos;
          changed |= nw != c;
          c = nw;
          c1 = c;
          s_choice[idx] = static_cast<uint8_t>(c);
        }
      }
      // the wave's own row of chunk counts and the block's counts: a token
      // that changed its choice moves one count (round 0: every row cleared
      // first; a wave's LDS operations complete in order)
      int* row = s_cc[u * kXWaves + wave];
      if (round == 0) {
        if (lane < G) row[lane] = 0;
        __builtin_amdgcn_wave_barrier();
      }
      if (c != c0) {
        if (c0 < G) {
          atomicSub(&row[c0], 1);
          atomicSub(&s_cnt[c0], 1);
        }
        if (c < G) {
          atomicAdd(&row[c], 1);
          atomicAdd(&s_cnt[c], 1);
        }
      }
    }
    const int any = __syncthreads_or(changed);
    // 2. (wave 0) publish this block's counts and whether any of its tokens
    // changed; 3. then every block's flag of the previous round (the flags
    // are 0 or 1: their sum is nonzero when any is set)
    if (wave == 0) {
      if (lane < G) {
        const int c = s_cnt[lane];
        __hip_atomic_store(xr + static_cast<int64_t>(b) * words + lane,
                           xword(round, static_cast<uint32_t>(c)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0)
        __hip_atomic_store(xr + static_cast<int64_t>(b) * words + G,
                           xword(round, static_cast<uint32_t>(any)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      int ch = 1, ok = 1;
      if (round > 0) {
        const uint64_t* xp = rec + static_cast<int64_t>((round - 1) % kXSlots) * nb * words;
        ok = xsum(xp + G, words, lane, kWave, nb, round - 1, ch) ? 1 : 0;
      }
      ch = ballot(ch != 0) != 0;
      ok = ballot(!ok) == 0;
      if (lane == 0) {
        s_changed = ch;
        if (!ok) s_abort = 1;
      }
    }
    // 4. counts of the blocks before this one: thread (c, r) adds rank r's
    // counts of blocks c, c + ng, ... below b
    {
      const int c = tid / MOE_MAX_G, r = tid % MOE_MAX_G;
      int pre = 0;
      if (r < G) {
        if (!xsum(xr + r, words, c, ng, b, round, pre))
          s_abort = 1;
        else if (pre != 0)
          atomicAdd(&s_pre[par][r], pre);
      }
    }
    __syncthreads();
    if (s_abort) {
      if (tid == 0) report(d_err, MOE_DERR_SYNC);
      return;
    }
    // No token of any block changed in the previous round: this round's
    // choices and counts repeat it, so they are the fixed point.
    const bool last = !s_changed || round + 1 == max_rounds;
    // 5. (every wave) the tokens each rank took in earlier blocks (lane = rank)
    P = lane < G ? s_pre[par][lane] : 0;
    if (last) break;
    // 6. the ranks open for the whole block, and those whose cap-th taker
    // lies inside it; each wave places some of the latter: the chunk from a
    // scan of the chunk counts (lane = chunk), the lane from the chunk's
    // ballot of that rank
    {
      const int cnt = lane < G ? s_cnt[lane] : 0;
      const bool open = lane < G && P + cnt < cap;
      const bool cross = lane < G && P < cap && P + cnt >= cap;
      if (wave == 0 && lane < G && !cross) s_lim[lane] = open ? INT_MAX : -1;
      uint64_t cm = ballot(cross);
      for (int i = 0; cm != 0; ++i, cm &= cm - 1) {
        if (i % kXWaves != wave) continue;
        const int rr = __ffsll(static_cast<long long>(cm)) - 1;
        const int need = cap - __builtin_amdgcn_readlane(P, rr);
        const int n = lane < nchunks ? s_cc[lane][rr] : 0;
        const int incl = wave_incl_scan(n);
        const uint64_t hit = ballot(lane < nchunks && incl >= need);
        const int q = __ffsll(static_cast<long long>(hit)) - 1;
        const int rest = need - (lane_value(incl, q) - lane_value(n, q));
        const int base = (q / kXWaves) * kXThreads + (q % kXWaves) * kWave;
        const uint64_t mm = ballot(s_choice[base + lane] == rr);
        const bool at = ((mm >> lane) & 1ull) && lanes_below(mm) == rest - 1;
        const uint64_t am = ballot(at);
        if (lane == 0) s_lim[rr] = t0 + base + (__ffsll(static_cast<long long>(am)) - 1);
      }
    }
    __syncthreads();
  }

  // Positions: the rank's shard offset r * cap + its tokens in earlier blocks
  // + in earlier chunks of this block + those before the token in its chunk.
  // Each wave turns the chunk counts of a sixteenth of the ranks into first
  // positions (lane = chunk).
  for (int r = wave; r < G; r += kXWaves) {
    const int n = lane < nchunks ? s_cc[lane][r] : 0;
    const int excl = wave_incl_scan(n) - n;
    if (lane < nchunks) s_cc[lane][r] = r * cap + __builtin_amdgcn_readlane(P, r) + excl;
  }
  __syncthreads();
  if (b == 0 && tid <= G) shard_offsets[tid] = tid * cap;
  for (int u = 0; u < tpt; ++u) {
    const int t = t0 + u * kXThreads + tid;
    const int c = s_choice[u * kXThreads + tid];
    // lanes before this one with the same rank: one ballot per distinct rank
    int below = 0;
    uint64_t rest = ballot(t < T && c < G);
    while (rest != 0) {
      const int v = lane_value(c, __ffsll(static_cast<long long>(rest)) - 1);
      const uint64_t m = ballot(c == v);
      if (c == v) below = lanes_below(m);
      rest &= ~m;
    }
    if (t < T) {
      const int pos = s_cc[u * kXWaves + wave][c] + below;
      pred_rank[t] = c;
      dest_pos[t] = pos;
      if (perm != nullptr) perm[pos] = t;
    }
  }
}

// Launch shape of the exchange form for T tokens, or ok = false when it does
// not apply (no tokens, more than kXBlocks * kXThreads * kXMaxTpt tokens, or
// more blocks than the device holds at once, which the blocks' waits on each
// other need): then the round-per-launch kernels and the plan's sort run.
struct XShape {
  bool ok;
  int tpt, TB, nb;
};

std::mutex g_xres_mu;
int g_xres[64] = {};  // blocks of the exchange kernel the device holds at once, per device

int exchange_residency() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(g_xres_mu);
  if (g_xres[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    // the fewest blocks per CU over the kernel's instances
    const void* kernels[] = {reinterpret_cast<const void*>(shuffle_exchange_kernel<1>),
                             reinterpret_cast<const void*>(shuffle_exchange_kernel<2>),
                             reinterpret_cast<const void*>(shuffle_exchange_kernel<3>),
                             reinterpret_cast<const void*>(shuffle_exchange_kernel<4>)};
    per_cu = INT32_MAX;
    for (const void* kern : kernels) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kXThreads, 0) != hipSuccess)
        return 0;
      per_cu = n < per_cu ? n : per_cu;
    }
    g_xres[dev] = per_cu * cus;
  }
  return g_xres[dev];
}

XShape exchange_shape(int64_t T) {
  XShape x{false, 0, 0, 0};
  if (T <= 0) return x;
  const int64_t per_pass = static_cast<int64_t>(kXBlocks) * kXThreads;
  const int64_t tpt = (T + per_pass - 1) / per_pass;
  if (tpt > kXMaxTpt) return x;
  x.tpt = static_cast<int>(tpt);
  x.TB = x.tpt * kXThreads;
  x.nb = static_cast<int>((T + x.TB - 1) / x.TB);
  x.ok = x.nb <= exchange_residency();
  return x;
}

struct BalancedWs {
  ShuffleWs base;
  int64_t* scores;
  int32_t* fill_hist;  // [2][G]: the fill indices of the last two rounds
  int32_t* flag;
  int32_t* tile_cnt;   // [2][NT][G]
  uint64_t* tile_mask; // [2][NT][G][waves per tile]
  uint8_t* prefs;      // [T][pref_stride(G)]: each token's ranks in preference order
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
  w.prefs = reinterpret_cast<uint8_t*>(take(static_cast<size_t>(T > 0 ? T : 1) * pref_stride(G)));
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
  const moe::XShape xs = moe::exchange_shape(T);
  if (xs.ok) {
    const int64_t Gs = moe::pref_stride(G);
    const int64_t rec_words = static_cast<int64_t>(moe::kXSlots) * xs.nb * (G + 1);
    const int W = moe::group_width(G);
    const int per_block = 256 / W * moe::kScoreTokens;
    auto sort = [&](auto kernel) {
      kernel<<<(Ti + per_block - 1) / per_block, 256, 0, s>>>(topk, Ti, k, E, w.base.M, G, Gs,
                                                            w.prefs, w.base.rec, rec_words, d_err);
    };
    switch (W) {
      case 1: sort(moe::prefs_sort_kernel<1>); break;
      case 2: sort(moe::prefs_sort_kernel<2>); break;
      case 4: sort(moe::prefs_sort_kernel<4>); break;
      case 8: sort(moe::prefs_sort_kernel<8>); break;
      case 16: sort(moe::prefs_sort_kernel<16>); break;
      case 32: sort(moe::prefs_sort_kernel<32>); break;
      default: sort(moe::prefs_sort_kernel<64>); break;
    }
    MOE_CHECK_LAUNCH();
    const int pwords = static_cast<int>(Gs / 16);
    auto launch = [&](auto kernel) {
      kernel<<<xs.nb, moe::kXThreads, 0, s>>>(w.prefs, Gs, Ti, G, Ti / G, xs.TB, xs.tpt, xs.nb,
                                              w.base.rec, pred_rank, dest_pos, perm,
                                              shard_offsets, d_err);
    };
    if (pwords == 1)
      launch(moe::shuffle_exchange_kernel<1>);
    else if (pwords == 2)
      launch(moe::shuffle_exchange_kernel<2>);
    else if (pwords == 3)
      launch(moe::shuffle_exchange_kernel<3>);
    else
      launch(moe::shuffle_exchange_kernel<4>);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
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
  // The prediction: for up to 16 ranks, fused with the sort's tile counts
  // (predict_count_kernel below); above, a group of lanes per token reads the
  // token's rows of M coalesced (rank_argmax_kernel) and the plan's count
  // kernel takes the tile counts.  Neither waits on other blocks, so the
  // prediction can run beside other kernels.
  if (G > 16 && Ti > 0) {
    const int W = moe::group_width(G);
    const int per_block = 256 / W * moe::kScoreTokens;
    if (W == 32)
      moe::rank_argmax_kernel<32><<<(Ti + per_block - 1) / per_block, 256, 0, s>>>(
          topk, Ti, k, E, w.M, G, pred_rank, w.rec, 0, d_err);
    else
      moe::rank_argmax_kernel<64><<<(Ti + per_block - 1) / per_block, 256, 0, s>>>(
          topk, Ti, k, E, w.M, G, pred_rank, w.rec, 0, d_err);
    MOE_CHECK_LAUNCH();
    moe::PlanArgs a{pred_rank,      nullptr,        Ti,        1,
                    G,              w.identity,     G,         G,
                    w.src1,         T,              w.send_counts, w.send_offsets,
                    perm ? perm : w.perm_scratch,   nullptr,   dest_pos,
                    nullptr,        w.counters,     d_err,     w.plan_ws,
                    shard_offsets};
    return moe::launch_plan(a, s);
  }
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
