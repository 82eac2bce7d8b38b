// Destination-side expert layout.
//
// On each destination rank the received token rows are expanded into one
// row per (token, expert) assignment, grouped per local expert -- the layout
// a grouped expert GEMM consumes ("Training Communication-Efficient
// Mixture-of-Experts Language Models with Layer Re-Configuration": alltoall
// dispatch followed by grouped GEMM; footnote 3: the routed probabilities
// travel with the rows).  Rows are ordered by (rank p(e), expert e, token t).
//
// The order is a stable counting sort of the T*k assignments by expert, with
// experts taken in (rank, id) order.  Three kernels:
//   count : one block per 256-token tile; each expert's tokens in the tile
//           form a 256-bit column in LDS (atomic OR of one bit per slot);
//           popcounts give per-(tile, expert) counts.  Also fills row_dest
//           with -1.
//   scan  : one block; per expert the exclusive prefix over tiles; expert
//           blocks placed in (rank, id) order.
//   write : same tiles and columns; a slot's row is its expert's first row
//           plus the tile's prefix plus the popcount of its column below its
//           token.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kExTile = 256;
constexpr int kExWords = kExTile / 64;

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

inline int64_t ex_tiles(int64_t T) { return (T + kExTile - 1) / kExTile; }

// Builds the tile's expert columns; returns this thread's validated expert
// ids (-1 where skipped) and their ranks.
__device__ __forceinline__ int build_columns(const int32_t* __restrict__ topk, int T, int k, int E,
                                             const int32_t* __restrict__ expert_rank, int G,
                                             uint64_t (*cols)[kExWords], int (&ex)[MOE_MAX_K],
                                             int (&rk)[MOE_MAX_K]) {
  for (int i = threadIdx.x; i < E * kExWords; i += kExTile) (&cols[0][0])[i] = 0ull;
  __syncthreads();
  const int local = threadIdx.x;
  const int t = blockIdx.x * kExTile + local;
  int err = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    ex[j] = -1;
    rk[j] = -1;
    if (t < T && j < k) {
      const int e = topk[static_cast<int64_t>(t) * k + j];
      if (e < 0 || e >= E) {
        err |= MOE_DERR_EXPERT_RANGE;
        continue;
      }
#pragma unroll
      for (int q = 0; q < j; ++q)
        if (ex[q] == e) err |= MOE_DERR_EXPERT_DUP;
      const int r = expert_rank[e];
      if (r < 0 || r >= G) {
        err |= MOE_DERR_RANK_RANGE;
        continue;
      }
      ex[j] = e;
      rk[j] = r;
      atomicOr(reinterpret_cast<unsigned long long*>(&cols[e][local >> 6]),
               static_cast<unsigned long long>(1ull << (local & 63)));
    }
  }
  __syncthreads();
  return err;
}

__global__ __launch_bounds__(kExTile) void expert_count_kernel(
    const int32_t* __restrict__ topk, int T, int k, int E, const int32_t* __restrict__ expert_rank,
    int G, int32_t* __restrict__ tile_cnt, int32_t* __restrict__ row_dest, int64_t row_dest_n,
    int32_t* d_err) {
  __shared__ uint64_t cols[MOE_MAX_E][kExWords];
  // Part of the -1 fill of row_dest (the write kernel runs after this one).
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kExTile) + threadIdx.x; i < row_dest_n;
       i += static_cast<int64_t>(gridDim.x) * kExTile)
    row_dest[i] = -1;
  int ex[MOE_MAX_K], rk[MOE_MAX_K];
  const int err = build_columns(topk, T, k, E, expert_rank, G, cols, ex, rk);
  report(d_err, err);
  for (int e = threadIdx.x; e < E; e += kExTile) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kExWords; ++w) c += __popcll(cols[e][w]);
    tile_cnt[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] = c;
  }
}

constexpr int kExScanThreads = 1024;
constexpr int kExScanWaves = kExScanThreads / kWave;

__global__ __launch_bounds__(kExScanThreads) void expert_scan_kernel(
    int NT, int E, const int32_t* __restrict__ expert_rank, int G, int32_t* __restrict__ tile_cnt,
    int32_t* __restrict__ expert_first, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ rank_offsets) {
  __shared__ int s_count[MOE_MAX_E];
  __shared__ int s_rank[MOE_MAX_E];
  __shared__ int s_rtot[MOE_MAX_G + 1];
  __shared__ int s_roff[MOE_MAX_G + 1];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  for (int e = tid; e < E; e += kExScanThreads) {
    const int r = expert_rank[e];
    s_rank[e] = (r >= 0 && r < G) ? r : G;  // unplaced experts sort last, hold no rows
  }
  // Per expert: exclusive prefix of its tile counts, and its total.  The
  // loads of every chunk of the wave's next expert are issued before its
  // scan (kPre chunks of 64 tiles at once), so latencies overlap.
  constexpr int kPre = 8;
  for (int e = wave; e < E; e += kExScanWaves) {
    int pre[kPre];
#pragma unroll
    for (int c = 0; c < kPre; ++c) {
      const int j = c * kWave + lane;
      pre[c] = j < NT ? tile_cnt[static_cast<int64_t>(e) * NT + j] : 0;
    }
    int carry = 0;
#pragma unroll
    for (int c = 0; c < kPre; ++c) {
      if (c * kWave >= NT) break;
      const int j = c * kWave + lane;
      const int incl = wave_incl_scan(pre[c]) + carry;
      if (j < NT) tile_cnt[static_cast<int64_t>(e) * NT + j] = incl - pre[c];
      carry = lane_value(incl, kWave - 1);
    }
    for (int base = kPre * kWave; base < NT; base += kWave) {
      const int j = base + lane;
      const int v = j < NT ? tile_cnt[static_cast<int64_t>(e) * NT + j] : 0;
      const int incl = wave_incl_scan(v) + carry;
      if (j < NT) tile_cnt[static_cast<int64_t>(e) * NT + j] = incl - v;
      carry = lane_value(incl, kWave - 1);
    }
    if (lane == 0) s_count[e] = carry;
  }
  __syncthreads();
  // Expert blocks in (rank, id) order: rank totals by LDS atomics, a scan
  // over ranks, then each expert's offset inside its rank as the sum of the
  // counts of lower-id experts of the same rank (tpe threads per expert).
  if (tid <= G) s_rtot[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += kExScanThreads)
    if (s_rank[e] < G) atomicAdd(&s_rtot[s_rank[e]], s_count[e]);
  __syncthreads();
  if (wave == 0) {
    const int v = lane < G ? s_rtot[lane] : 0;
    const int incl = wave_incl_scan(v);
    if (lane < G) s_roff[lane] = incl - v;
    if (lane == 0) s_roff[G] = lane_value(incl, kWave - 1);
  }
  __syncthreads();
  int tpe = kExScanThreads / E;
  tpe = tpe >= 64 ? 64 : (tpe >= 32 ? 32 : (tpe >= 16 ? 16 : (tpe >= 8 ? 8 : (tpe >= 4 ? 4 : (tpe >= 2 ? 2 : 1)))));
  for (int base = 0; base < E * tpe; base += kExScanThreads) {
    const int g = base + tid;
    const int e = g / tpe, sub = g % tpe;
    int part = 0;
    if (e < E) {
      const int re = s_rank[e];
      for (int f = sub; f < e; f += tpe)
        if (s_rank[f] == re) part += s_count[f];
    }
    for (int d = tpe >> 1; d >= 1; d >>= 1) part += __shfl_xor(part, d, kWave);
    if (e < E && sub == 0) {
      const int re = s_rank[e];
      const int first = (re < G ? s_roff[re] : s_roff[G]) + part;
      expert_first[e] = first;
      expert_count[e] = s_count[e];
    }
  }
  for (int r = tid; r <= G; r += kExScanThreads) rank_offsets[r] = s_roff[r];
}

__global__ __launch_bounds__(kExTile) void expert_write_kernel(
    const int32_t* __restrict__ topk, const float* __restrict__ gates, int T, int k, int E,
    const int32_t* __restrict__ expert_rank, int G, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ expert_first, const int32_t* __restrict__ slot_row,
    int64_t send_rows, int32_t* __restrict__ erow,
    float* __restrict__ erow_weight, int32_t* __restrict__ erow_slot,
    int32_t* __restrict__ erow_src, int32_t* __restrict__ row_dest, int32_t* d_err) {
  __shared__ uint64_t cols[MOE_MAX_E][kExWords];
  int ex[MOE_MAX_K], rk[MOE_MAX_K];
  build_columns(topk, T, k, E, expert_rank, G, cols, ex, rk);
  const int local = threadIdx.x;
  const int t = blockIdx.x * kExTile + local;
  if (t >= T) return;
  const int word = local >> 6;
  const uint64_t below = (1ull << (local & 63)) - 1ull;
  int errbits = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (j >= k) break;
    const int64_t slot = static_cast<int64_t>(t) * k + j;
    if (ex[j] < 0) {
      erow[slot] = -1;
      continue;
    }
    const int e = ex[j];
    int pos = __popcll(cols[e][word] & below);
    for (int w = 0; w < word; ++w) pos += __popcll(cols[e][w]);
    const int row = expert_first[e] + tile_base[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] + pos;
    erow[slot] = row;
    if (erow_weight != nullptr) erow_weight[row] = gates != nullptr ? gates[slot] : 0.f;
    if (erow_slot != nullptr) erow_slot[row] = static_cast<int32_t>(slot);
    // Position of this slot among the token's slots on the same rank.
    int q = 0;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) q += (rk[jj] == rk[j]);
    const int i = slot_row[slot];
    const bool ok = i >= 0 && i < send_rows;
    if (ok)
      row_dest[static_cast<int64_t>(i) * k + q] = row;
    else
      errbits |= MOE_DERR_ROW_RANGE;
    if (erow_src != nullptr) erow_src[row] = ok ? i : -1;
  }
  report(d_err, errbits);
}

}  // namespace
}  // namespace moe

extern "C" int moe_expert_plan_workspace_size(int64_t T, int E, size_t* ws_bytes) {
  if (ws_bytes == nullptr) return MOE_ERR_NULL;
  if (T < 0 || E < 1 || E > MOE_MAX_E) return MOE_ERR_SHAPE;
  const int64_t nt = moe::ex_tiles(T) > 0 ? moe::ex_tiles(T) : 1;
  *ws_bytes = moe::align256(static_cast<size_t>(nt) * E * sizeof(int32_t));
  return MOE_OK;
}

extern "C" int moe_expert_plan(const int32_t* topk, const float* gates, int64_t T, int k, int E,
                               const int32_t* expert_rank, int G, const int32_t* slot_row,
                               int64_t send_rows, int32_t* erow, int32_t* expert_first,
                               int32_t* expert_count, int32_t* rank_offsets, float* erow_weight,
                               int32_t* erow_slot, int32_t* erow_src, int32_t* row_dest,
                               int32_t* d_err, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_E || G < 1 || G > MOE_MAX_G ||
      send_rows < 0 || T * static_cast<int64_t>(k) >= (int64_t{1} << 31) ||
      send_rows * static_cast<int64_t>(k) >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  if (expert_rank == nullptr || expert_first == nullptr || expert_count == nullptr ||
      rank_offsets == nullptr || ws == nullptr)
    return MOE_ERR_NULL;
  if (T > 0 && (topk == nullptr || slot_row == nullptr || erow == nullptr)) return MOE_ERR_NULL;
  if (send_rows > 0 && row_dest == nullptr) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return MOE_ERR_ALIGN;
  size_t need = 0;
  moe_expert_plan_workspace_size(T, E, &need);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Ti = static_cast<int>(T);
  const int NT = static_cast<int>(moe::ex_tiles(T));
  int32_t* tile_cnt = static_cast<int32_t*>(ws);
  // At least one block, so that row_dest is filled even without tokens.
  moe::expert_count_kernel<<<NT > 0 ? NT : 1, moe::kExTile, 0, s>>>(
      topk, Ti, k, E, expert_rank, G, tile_cnt, row_dest, send_rows * k, d_err);
  MOE_CHECK_LAUNCH();
  moe::expert_scan_kernel<<<1, moe::kExScanThreads, 0, s>>>(NT, E, expert_rank, G, tile_cnt,
                                                            expert_first, expert_count,
                                                            rank_offsets);
  MOE_CHECK_LAUNCH();
  if (NT > 0) {
    moe::expert_write_kernel<<<NT, moe::kExTile, 0, s>>>(topk, gates, Ti, k, E, expert_rank, G,
                                                          tile_cnt, expert_first, slot_row,
                                                          send_rows, erow, erow_weight, erow_slot,
                                                          erow_src, row_dest, d_err);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}
