// Internal launcher of the dispatch-plan kernels, shared by the plan entry
// point and by the token shuffle (which is a plan with one source rank,
// one "expert" per token and the identity placement: a stable counting sort).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kPlanTile = 256;  // tokens per tile = threads per block

// Upper bound of the number of token tiles: sum_s ceil(len_s / tile).
inline int64_t plan_max_tiles(int64_t T, int G) { return (T + kPlanTile - 1) / kPlanTile + G; }

inline size_t plan_workspace_bytes(int64_t T, int G) {
  const int64_t nt = plan_max_tiles(T, G);
  size_t b = static_cast<size_t>(nt) * (G + 4) * sizeof(int32_t);
  return (b + 255) & ~static_cast<size_t>(255);
}

// Where the count kernel leaves its per-tile results in the plan workspace:
// counts per (rank, tile) at cnt[r * stride + tile], then four counter
// partials per tile.
struct PlanTiles {
  int32_t* cnt;
  int32_t* stats;
  int64_t stride;
};

inline PlanTiles plan_tiles(void* ws, int64_t T, int G) {
  const int64_t nt = plan_max_tiles(T, G);
  int32_t* cnt = static_cast<int32_t*>(ws);
  return PlanTiles{cnt, cnt + nt * G, nt};
}

struct PlanArgs {
  const int32_t* topk;
  const float* gates;
  int T, k, E;
  const int32_t* expert_rank;
  int G, ranks_per_node;
  const int32_t* src_offsets;
  int64_t row_capacity;
  int32_t* send_counts;
  int32_t* send_offsets;
  int32_t* row_token;
  float* row_weight;
  int32_t* token_rows;
  int32_t* slot_row;
  int64_t* counters;
  int32_t* d_err;
  void* ws;
  // Optional: receives send_offsets[0..G] (the row offsets of source rank 0's
  // blocks), i.e. the bucket offsets when the plan serves as a sort.
  int32_t* first_offsets = nullptr;
  // Set when the per-tile counts are already in the workspace (the token
  // shuffle's prediction kernel writes them): the count kernel is skipped.
  bool counts_ready = false;
  // Optional: plan the batch in the order perm (position p holds token
  // perm[p] of topk / gates); the count kernel then writes that order's
  // routing to topk_out / gates_out, which the write kernel reads.
  const int32_t* perm = nullptr;
  int32_t* topk_out = nullptr;
  float* gates_out = nullptr;
};

// Enqueues the three plan kernels; arguments already validated.
int launch_plan(const PlanArgs& a, hipStream_t stream);

}  // namespace moe
