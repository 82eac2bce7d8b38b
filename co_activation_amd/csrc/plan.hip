// Deduplicated dispatch plan.
//
// "Expert Coupling in MoE Pretraining ..." (abstract): deduplicated dispatch,
// a token reaches a given GPU at most one time however many of its experts
// live there.  "Cobalt: Leveraging Expert Co-activation ..."
// (Problem Formulation): token t with expert set D_t on source rank s_t; with
// one replica per expert the rank of (t, e) is p(e); cross-node volume
// V = sum_t |{N(p(e)) : e in D_t} minus {N(s_t)}|.
//
// Rows are ordered by (source rank s, destination rank r, token t).  A token
// is a 64-bit mask of its destination ranks (G <= 64 = wave width).  Three
// kernels:
//   count : one block per 256-token tile that never straddles two source
//           ranks; per-rank counts of the tile from wave ballots, plus the
//           tile's counter partials.  No atomics, so the result is exact and
//           order independent.
//   scan  : one block; per rank a segmented scan over the tiles of each
//           source rank (rank r's tiles are walked by one wave 64 at a time),
//           then an exclusive scan of S[s][r] in (s, r) order; per tile it
//           leaves the prefix inside its (s, r) block.
//   write : one block per tile; the same ballots give each token's position
//           inside its wave, LDS gives the wave's offset inside the tile.
#include <mutex>

#include "plan.hpp"

namespace moe {
namespace {

// Lane s (< G) receives source rank s's token range [lo, hi), the index of
// its first tile and the inclusive tile prefix; every lane receives the total
// tile count.  Offsets that are not a partition of [0, T) are repaired into
// one (clamped, made nondecreasing, first = 0, last = T) so that every access
// stays in bounds, and MOE_DERR_SRC_OFFSETS is returned.
__device__ __forceinline__ int load_shards(const int32_t* off, int T, int G, int& lo, int& hi,
                                           int& first, int& incl, int& total) {
  const int lane = lane_id();
  bool bad = false;
  int ca, cb;
  if (off == nullptr) {
    const int per = T / G;
    ca = min(lane, G) * per;
    cb = min(lane + 1, G) * per;
  } else {
    const int ra = lane < G ? off[lane] : T;
    const int rb = lane < G ? off[lane + 1] : T;
    bad = lane < G && (ra < 0 || rb > T || rb < ra || (lane == 0 && ra != 0) ||
                       (lane == G - 1 && rb != T));
    ca = min(max(ra, 0), T);
    cb = min(max(rb, 0), T);
    if (lane == 0) ca = 0;
    if (lane >= G - 1) cb = T;
    ca = wave_incl_max(ca);
    cb = max(ca, cb);
  }
  lo = ca;
  hi = cb;
  const int nt = lane < G ? (hi - lo + kPlanTile - 1) / kPlanTile : 0;
  incl = wave_incl_scan(nt);
  first = incl - nt;
  total = lane_value(incl, kWave - 1);
  return ballot(bad) ? MOE_DERR_SRC_OFFSETS : 0;
}

// The tile handled by this block: source rank s and tokens [t0, t1).
// Returns false when the block index is past the last tile.
__device__ __forceinline__ bool block_tile(const int32_t* off, int T, int G, int& s, int& t0,
                                           int& t1, int& err) {
  int lo, hi, first, incl, total;
  err = load_shards(off, T, G, lo, hi, first, incl, total);
  const int j = blockIdx.x;
  if (j >= total) return false;
  s = __popcll(ballot(lane_id() < G && incl <= j));
  const int s_lo = lane_value(lo, s);
  const int s_hi = lane_value(hi, s);
  const int s_first = lane_value(first, s);
  t0 = s_lo + (j - s_first) * kPlanTile;
  t1 = min(t0 + kPlanTile, s_hi);
  return true;
}

// With perm set, position t of the plan holds token perm[t]: its routing
// is read through perm and copied to topk_out / gates_out (row t), so the
// gathered routing comes out of this pass.
__global__ __launch_bounds__(kPlanTile) void plan_count_kernel(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ perm,
    const float* __restrict__ gates, int32_t* __restrict__ topk_out,
    float* __restrict__ gates_out, int T, int k, int E, const int32_t* __restrict__ expert_rank,
    int G, int ranks_per_node, const int32_t* __restrict__ src_offsets,
    int32_t* __restrict__ tile_cnt, int64_t stride, int32_t* __restrict__ tile_stats,
    int32_t* d_err) {
  __shared__ int s_cnt[kPlanTile / kWave][kWave];
  __shared__ int s_stat[kPlanTile / kWave][4];
  const int lane = lane_id();
  const int wave = wave_id();
  int s, t0, t1, off_err;
  if (!block_tile(src_offsets, T, G, s, t0, t1, off_err)) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) report(d_err, off_err);

  const int t = t0 + static_cast<int>(threadIdx.x);
  uint64_t mask = 0, nodes = 0;
  int local_assign = 0, errbits = 0;
  int src = t;
  if (t < t1 && perm != nullptr) {
    src = perm[t];
    if (src < 0 || src >= T) {
      errbits |= MOE_DERR_ROW_RANGE;
      src = -1;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (j >= k) break;
      const int64_t i = static_cast<int64_t>(src) * k + j;
      topk_out[static_cast<int64_t>(t) * k + j] = src >= 0 ? topk[i] : -1;
      if (gates_out != nullptr)
        gates_out[static_cast<int64_t>(t) * k + j] = (src >= 0 && gates != nullptr) ? gates[i] : 0.f;
    }
  }
  if (t < t1 && src >= 0) {
    const int32_t* row = topk + static_cast<int64_t>(src) * k;
    // every id load, then every rank lookup, goes out before any is used
    int ex[MOE_MAX_K], rk[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) ex[j] = j < k ? row[j] : -1;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j)
      rk[j] = (j < k && ex[j] >= 0 && ex[j] < E) ? expert_rank[ex[j]] : -1;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (j >= k) break;
      const int e = ex[j];
#pragma unroll
      for (int q = 0; q < j; ++q)
        if (ex[q] == e) errbits |= MOE_DERR_EXPERT_DUP;
      if (e < 0 || e >= E) {
        errbits |= MOE_DERR_EXPERT_RANGE;
        continue;
      }
      const int r = rk[j];
      if (r < 0 || r >= G) {
        errbits |= MOE_DERR_RANK_RANGE;
        continue;
      }
      mask |= 1ull << r;
      nodes |= 1ull << (r / ranks_per_node);
      local_assign += (r == s);
    }
  }
  report(d_err, errbits);

  int mine = 0;
  for (int r = 0; r < G; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (lane == r) mine = __popcll(b);
  }
  if (lane < G) s_cnt[wave][lane] = mine;

  const int local_row = static_cast<int>((mask >> s) & 1ull);
  const int node_rows = __popcll(nodes);
  const int cross = __popcll(nodes & ~(1ull << (s / ranks_per_node)));
  const int v0 = wave_sum(local_row), v1 = wave_sum(local_assign);
  const int v2 = wave_sum(node_rows), v3 = wave_sum(cross);
  if (lane == 0) {
    s_stat[wave][0] = v0;
    s_stat[wave][1] = v1;
    s_stat[wave][2] = v2;
    s_stat[wave][3] = v3;
  }
  __syncthreads();
  const int j = blockIdx.x;
  if (threadIdx.x < static_cast<unsigned>(G)) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPlanTile / kWave; ++w) c += s_cnt[w][threadIdx.x];
    tile_cnt[static_cast<int64_t>(threadIdx.x) * stride + j] = c;
  }
  if (threadIdx.x < 4) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPlanTile / kWave; ++w) c += s_stat[w][threadIdx.x];
    tile_stats[static_cast<int64_t>(j) * 4 + threadIdx.x] = c;
  }
}

// Smallest s in [0, G) with incl[s] > j (the source rank of tile j).
__device__ __forceinline__ int shard_of_tile(int j, const int* incl, int G) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > j)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// kScanThreads is 256 for up to 16 ranks and 1024 above: a four-wave block
// finds room on a CU that a bandwidth-bound kernel on another stream keeps
// full far sooner than a sixteen-wave one.
template <int kScanThreads>
__global__ __launch_bounds__(kScanThreads) void plan_scan_kernel(
    const int32_t* __restrict__ src_offsets, int T, int k, int G, int32_t* __restrict__ tile_cnt,
    int64_t stride, const int32_t* __restrict__ tile_stats, int64_t row_capacity, int32_t* __restrict__ send_counts,
    int32_t* __restrict__ send_offsets, int64_t* __restrict__ counters,
    int32_t* __restrict__ first_offsets, int32_t* d_err) {
  constexpr int kScanWaves = kScanThreads / kWave;
  constexpr int kPer = MOE_MAX_G * MOE_MAX_G / kScanThreads;  // S entries per thread
  __shared__ int s_incl[kWave];
  __shared__ int s_first[kWave];
  __shared__ int s_S[MOE_MAX_G * MOE_MAX_G];
  __shared__ int s_part[kScanWaves];
  __shared__ long long s_red[kScanWaves][4];
  __shared__ int s_maxrecv;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();

  int lo, hi, first, incl, NT;
  load_shards(src_offsets, T, G, lo, hi, first, incl, NT);
  if (wave == 0) {
    s_incl[lane] = incl;
    s_first[lane] = first;
  }
  for (int i = tid; i < G * G; i += kScanThreads) s_S[i] = 0;
  __syncthreads();

  // Per destination rank r: exclusive prefix of the tile counts within each
  // source rank (segments), and the segment totals S[s][r].  A wave takes
  // kGroup ranks at a time; the first kPrefetch chunks of 64 tiles of each
  // are loaded before any is scanned, so their load latencies overlap.
  constexpr int kPrefetch = 8;
  constexpr int kGroup = 4;
  for (int r0 = wave; r0 < G; r0 += kScanWaves * kGroup) {
    int pre[kGroup][kPrefetch];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int r = r0 + g * kScanWaves;
#pragma unroll
      for (int c = 0; c < kPrefetch; ++c) {
        const int j = c * kWave + lane;
        pre[g][c] = (r < G && j < NT) ? tile_cnt[static_cast<int64_t>(r) * stride + j] : 0;
      }
    }
    int carry[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) carry[g] = 0;
    for (int base = 0, c = 0; base < NT; base += kWave, ++c) {
      const int j = base + lane;
      const bool in = j < NT;
      const int s = in ? shard_of_tile(j, s_incl, G) : 0;
      const bool head = in && s_first[s] == j;
      const bool last = in && j + 1 == s_incl[s];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const int r = r0 + g * kScanWaves;  // uniform across the wave
        if (r >= G) break;
        int v = 0;
        if (c < kPrefetch) {
#pragma unroll
          for (int q = 0; q < kPrefetch; ++q)
            if (q == c) v = pre[g][q];
        } else if (in) {
          v = tile_cnt[static_cast<int64_t>(r) * stride + j];
        }
        int val = v;
        int flag = head ? 1 : 0;
        wave_seg_scan(val, flag);
        if (!flag) val += carry[g];
        if (in) tile_cnt[static_cast<int64_t>(r) * stride + j] = val - v;
        if (last) s_S[s * G + r] = val;
        carry[g] = lane_value(val, kWave - 1);
      }
    }
  }
  __syncthreads();

  // Rows received per destination rank; the largest one.
  if (wave == 0) {
    int col = 0;
    if (lane < G)
      for (int s = 0; s < G; ++s) col += s_S[s * G + lane];
    col = wave_max(col);
    if (lane == 0) s_maxrecv = col;
  }

  // Exclusive scan of S in (s, r) order: kPer consecutive entries per thread.
  const int n = G * G;
  const int i0 = tid * kPer;
  int v[kPer];
  int local = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    v[q] = (i0 + q < n) ? s_S[i0 + q] : 0;
    local += v[q];
  }
  const int winc = wave_incl_scan(local);
  if (lane == kWave - 1) s_part[wave] = winc;
  __syncthreads();
  if (wave == 0) {
    int p = lane < kScanWaves ? s_part[lane] : 0;
    p = wave_incl_scan(p);
    if (lane < kScanWaves) s_part[lane] = p;
  }
  __syncthreads();
  int run = (wave ? s_part[wave - 1] : 0) + winc - local;
  const int total_rows = s_part[kScanWaves - 1];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (i0 + q < n) {
      send_counts[i0 + q] = v[q];
      send_offsets[i0 + q] = run;
      s_S[i0 + q] = run;
      run += v[q];
    }
  }
  if (tid == 0) send_offsets[n] = total_rows;
  __syncthreads();
  if (first_offsets != nullptr && tid <= G) first_offsets[tid] = tid < n ? s_S[tid] : total_rows;

  // Counters.
  long long c[4] = {0, 0, 0, 0};
  for (int j = tid; j < NT; j += kScanThreads) {
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] += tile_stats[static_cast<int64_t>(j) * 4 + q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const long long w = wave_sum64(c[q]);
    if (lane == 0) s_red[wave][q] = w;
  }
  __syncthreads();
  if (tid < 4) {
    long long w = 0;
    for (int q = 0; q < kScanWaves; ++q) w += s_red[q][tid];
    counters[2 + tid] = w;
  }
  if (tid == 0) {
    counters[0] = total_rows;
    counters[1] = static_cast<long long>(T) * k;
    counters[6] = s_maxrecv;
    counters[7] = 0;
    if (static_cast<int64_t>(total_rows) > row_capacity) report(d_err, MOE_DERR_CAPACITY);
  }
}

__global__ __launch_bounds__(kPlanTile) void plan_write_kernel(
    const int32_t* __restrict__ topk, const float* __restrict__ gates, int T, int k, int E,
    const int32_t* __restrict__ expert_rank, int G, const int32_t* __restrict__ src_offsets,
    const int32_t* __restrict__ tile_base, int64_t stride,
    const int32_t* __restrict__ send_offsets, int64_t row_capacity,
    int32_t* __restrict__ row_token,
    float* __restrict__ row_weight, int32_t* __restrict__ token_rows,
    int32_t* __restrict__ slot_row, int32_t* d_err) {
  __shared__ int s_cnt[kPlanTile / kWave][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  int s, t0, t1, off_err;
  if (!block_tile(src_offsets, T, G, s, t0, t1, off_err)) return;

  const int t = t0 + static_cast<int>(threadIdx.x);
  const bool valid = t < t1;
  // every id and gate load, then every rank lookup, goes out before any is
  // used
  int ex[MOE_MAX_K], rk[MOE_MAX_K];
  float w[MOE_MAX_K];
  uint64_t mask = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    const bool in = valid && j < k;
    ex[j] = in ? topk[static_cast<int64_t>(t) * k + j] : -1;
    w[j] = (in && gates != nullptr) ? gates[static_cast<int64_t>(t) * k + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j)
    rk[j] = (ex[j] >= 0 && ex[j] < E) ? expert_rank[ex[j]] : -1;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (rk[j] < 0 || rk[j] >= G) rk[j] = -1;
    if (rk[j] >= 0) mask |= 1ull << rk[j];
  }

  int mine = 0;
  for (int r = 0; r < G; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (lane == r) mine = __popcll(b);
  }
  if (lane < G) s_cnt[wave][lane] = mine;
  __syncthreads();
  // First row of (this wave, rank = lane): the (s, r) block's offset, the
  // tile's prefix inside the block, the earlier waves of the tile.
  int mybase = 0;
  if (lane < G) {
    mybase = send_offsets[s * G + lane] + tile_base[static_cast<int64_t>(lane) * stride + blockIdx.x];
    for (int w2 = 0; w2 < wave; ++w2) mybase += s_cnt[w2][lane];
  }

  int32_t* trow = token_rows + static_cast<int64_t>(t) * k;
  int q = 0;
  int errbits = 0;
  for (int r = 0; r < G; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (b == 0) continue;
    const int rbase = lane_value(mybase, r);
    if ((mask >> r) & 1ull) {
      const int row = rbase + lanes_below(b);
      trow[q++] = row;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j) {
        if (j < k && rk[j] == r) {
          acc = acc + w[j];
          if (slot_row != nullptr) slot_row[static_cast<int64_t>(t) * k + j] = row;
        }
      }
      if (row < row_capacity) {
        row_token[row] = t;
        if (row_weight != nullptr) row_weight[row] = acc;
      } else {
        errbits |= MOE_DERR_CAPACITY;
      }
    }
  }
  if (valid) {
    for (int qq = q; qq < k; ++qq) trow[qq] = -1;
    if (slot_row != nullptr) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (j < k && rk[j] < 0) slot_row[static_cast<int64_t>(t) * k + j] = -1;
    }
  }
  report(d_err, errbits);
}

}  // namespace

int launch_plan(const PlanArgs& a, hipStream_t stream) {
  const PlanTiles tiles = plan_tiles(a.ws, a.T, a.G);
  const int64_t nt = tiles.stride;
  int32_t* tile_cnt = tiles.cnt;
  int32_t* tile_stats = tiles.stats;
  if (nt > 0 && !a.counts_ready) {
    plan_count_kernel<<<dim3(static_cast<unsigned>(nt)), dim3(kPlanTile), 0, stream>>>(
        a.topk, a.perm, a.gates, a.topk_out, a.gates_out, a.T, a.k, a.E, a.expert_rank, a.G,
        a.ranks_per_node, a.src_offsets, tile_cnt, nt, tile_stats, a.d_err);
    MOE_CHECK_LAUNCH();
  }
  if (a.G <= 16)
    plan_scan_kernel<256><<<dim3(1), dim3(256), 0, stream>>>(
        a.src_offsets, a.T, a.k, a.G, tile_cnt, nt, tile_stats, a.row_capacity, a.send_counts,
        a.send_offsets, a.counters, a.first_offsets, a.d_err);
  else
    plan_scan_kernel<1024><<<dim3(1), dim3(1024), 0, stream>>>(
        a.src_offsets, a.T, a.k, a.G, tile_cnt, nt, tile_stats, a.row_capacity, a.send_counts,
        a.send_offsets, a.counters, a.first_offsets, a.d_err);
  MOE_CHECK_LAUNCH();
  if (nt > 0) {
    // with perm, the routing in the plan's order is the count kernel's copy
    const int32_t* wtopk = a.perm != nullptr ? a.topk_out : a.topk;
    const float* wgates = a.perm != nullptr ? a.gates_out : a.gates;
    plan_write_kernel<<<dim3(static_cast<unsigned>(nt)), dim3(kPlanTile), 0, stream>>>(
        wtopk, wgates, a.T, a.k, a.E, a.expert_rank, a.G, a.src_offsets, tile_cnt, nt,
        a.send_offsets, a.row_capacity, a.row_token, a.row_weight, a.token_rows, a.slot_row,
        a.d_err);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}

}  // namespace moe

extern "C" int moe_dispatch_plan_workspace_size(int64_t T, int G, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return MOE_ERR_NULL;
  if (T < 0 || G < 1 || G > MOE_MAX_G) return MOE_ERR_SHAPE;
  *ws_bytes = moe::plan_workspace_bytes(T, G);
  return MOE_OK;
}

namespace moe {
namespace {

// Host checks of a plan call's sizes and pointers (the workspace aside).
int plan_check(const int32_t* topk, int64_t T, int k, int E, const int32_t* expert_rank, int G,
               int ranks_per_node, const int32_t* src_offsets, int64_t row_capacity,
               const int32_t* send_counts, const int32_t* send_offsets, const int32_t* row_token,
               const int32_t* token_rows, const int64_t* counters) {
  if (k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_E || G < 1 || G > MOE_MAX_G || T < 0 ||
      ranks_per_node < 1 || G % ranks_per_node != 0 || row_capacity < 0 ||
      row_capacity > INT32_MAX || T * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (src_offsets == nullptr && T % G != 0) return MOE_ERR_SHAPE;
  if (expert_rank == nullptr || send_counts == nullptr || send_offsets == nullptr ||
      counters == nullptr)
    return MOE_ERR_NULL;
  if (T > 0 && (topk == nullptr || token_rows == nullptr)) return MOE_ERR_NULL;
  if (row_capacity > 0 && row_token == nullptr) return MOE_ERR_NULL;
  return MOE_OK;
}

int plan_entry(const int32_t* topk, const float* gates, const int32_t* perm, int64_t T, int k,
               int E, const int32_t* expert_rank, int G, int ranks_per_node,
               const int32_t* src_offsets, int64_t row_capacity, int32_t* send_counts,
               int32_t* send_offsets, int32_t* row_token, float* row_weight,
               int32_t* token_rows, int32_t* slot_row, int64_t* counters, int32_t* topk_out,
               float* gates_out, int32_t* d_err, void* ws, size_t ws_bytes, void* stream) {
  const int st = plan_check(topk, T, k, E, expert_rank, G, ranks_per_node, src_offsets,
                            row_capacity, send_counts, send_offsets, row_token, token_rows,
                            counters);
  if (st != MOE_OK) return st;
  if (ws == nullptr) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return MOE_ERR_ALIGN;
  if (ws_bytes < plan_workspace_bytes(T, G)) return MOE_ERR_WORKSPACE;
  PlanArgs a{topk,         gates,        static_cast<int>(T), k,         E,
             expert_rank,  G,            ranks_per_node,      src_offsets, row_capacity,
             send_counts,  send_offsets, row_token,           row_weight, token_rows,
             slot_row,     counters,     d_err,               ws};
  a.perm = perm;
  a.topk_out = topk_out;
  a.gates_out = gates_out;
  return launch_plan(a, static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace moe

extern "C" int moe_dispatch_plan(const int32_t* topk, const float* gates, int64_t T, int k, int E,
                                 const int32_t* expert_rank, int G, int ranks_per_node,
                                 const int32_t* src_offsets, int64_t row_capacity,
                                 int32_t* send_counts, int32_t* send_offsets, int32_t* row_token,
                                 float* row_weight, int32_t* token_rows, int32_t* slot_row,
                                 int64_t* counters, int32_t* d_err, void* ws, size_t ws_bytes,
                                 void* stream) {
  return moe::plan_entry(topk, gates, nullptr, T, k, E, expert_rank, G, ranks_per_node,
                         src_offsets, row_capacity, send_counts, send_offsets, row_token,
                         row_weight, token_rows, slot_row, counters, nullptr, nullptr, d_err, ws,
                         ws_bytes, stream);
}

// ------------------------------------------------- no-allocation variant
//
// The plan's per-tile counts live in a device array of fixed size instead of
// a caller workspace, for callers that cannot allocate.  Every call on one
// device shares that device's copy of the array; the count kernel writes
// every entry the scan and write kernels then read, so nothing needs
// clearing between calls, but calls that overlap on one device race.

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The address of the current device's copy of `scratch`, looked up once per
// device.  (The array's name in host code is only a stand-in; kernels must
// be given this address.)
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_dispatch_plan_noalloc(const int32_t* topk, const float* gates, int64_t T,
                                         int k, int E, const int32_t* expert_rank, int G,
                                         int ranks_per_node, const int32_t* src_offsets,
                                         int64_t row_capacity, int32_t* send_counts,
                                         int32_t* send_offsets, int32_t* row_token,
                                         float* row_weight, int32_t* token_rows,
                                         int32_t* slot_row, int64_t* counters, int32_t* d_err,
                                         void* stream) {
  int st = moe::plan_check(topk, T, k, E, expert_rank, G, ranks_per_node, src_offsets,
                           row_capacity, send_counts, send_offsets, row_token, token_rows,
                           counters);
  if (st != MOE_OK) return st;
  if (moe::plan_workspace_bytes(T, G) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  st = moe::device_scratch(&ws);
  if (st != MOE_OK) return st;
  return moe::plan_entry(topk, gates, nullptr, T, k, E, expert_rank, G, ranks_per_node,
                         src_offsets, row_capacity, send_counts, send_offsets, row_token,
                         row_weight, token_rows, slot_row, counters, nullptr, nullptr, d_err, ws,
                         MOE_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int moe_dispatch_plan_gathered(
    const int32_t* topk, const float* gates, const int32_t* perm, int64_t T, int k, int E,
    const int32_t* expert_rank, int G, int ranks_per_node, const int32_t* src_offsets,
    int64_t row_capacity, int32_t* send_counts, int32_t* send_offsets, int32_t* row_token,
    float* row_weight, int32_t* token_rows, int32_t* slot_row, int64_t* counters,
    int32_t* topk_out, float* gates_out, int32_t* d_err, void* ws, size_t ws_bytes,
    void* stream) {
  if (T > 0 && (perm == nullptr || topk_out == nullptr || (gates != nullptr && gates_out == nullptr)))
    return MOE_ERR_NULL;
  if (T > 0 && (topk_out == topk || (gates_out != nullptr &&
                                     static_cast<const void*>(gates_out) == gates)))
    return MOE_ERR_SHAPE;
  return moe::plan_entry(topk, gates, perm, T, k, E, expert_rank, G, ranks_per_node, src_offsets,
                         row_capacity, send_counts, send_offsets, row_token, row_weight,
                         token_rows, slot_row, counters, topk_out, gates_out, d_err, ws, ws_bytes,
                         stream);
}
