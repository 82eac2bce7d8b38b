// Co-activation placement planner (host).
//
// "Expert Coupling in MoE Pretraining ..." (abstract): experts that are often
// selected together are placed on the same GPU.  "Cobalt: Leveraging Expert
// Co-activation for Efficient Distributed MoE Training" (Stage 1): the layout
// is re-planned from moving averages of co-selection counts and expert loads
// to keep co-activation inside ranks under a workload limit.  The pages give
// no algorithm; this grows one rank at a time: ranks 0..G-1 are filled in
// order, each step adding the unplaced expert most co-selected with the
// rank's experts so far (ties: larger total co-activation, then lower id, so
// an empty rank is seeded with the most co-activated expert left), preferring
// experts that keep the rank's load within (1 + eps) * total / G.  Sums are
// double precision over the float inputs, in ascending expert order.
#include <algorithm>
#include <vector>

#include "moe_coact.h"

extern "C" int moe_place_experts(const float* coact, const float* load, int E, int G, double eps,
                                 int32_t* expert_rank) {
  if (coact == nullptr || load == nullptr || expert_rank == nullptr) return MOE_ERR_NULL;
  if (E < 1 || E > MOE_MAX_E || G < 1 || G > MOE_MAX_G || E % G != 0 || !(eps >= 0.0))
    return MOE_ERR_SHAPE;
  const int cap = E / G;
  double total_load = 0.0;
  for (int e = 0; e < E; ++e) total_load += static_cast<double>(load[e]);
  const double limit = (1.0 + eps) * total_load / G;
  auto C = [&](int a, int b) { return static_cast<double>(coact[static_cast<size_t>(a) * E + b]); };

  std::vector<double> total(E, 0.0);
  for (int e = 0; e < E; ++e)
    for (int f = 0; f < E; ++f)
      if (f != e) total[e] += C(e, f);
  for (int e = 0; e < E; ++e) expert_rank[e] = -1;

  for (int r = 0; r < G; ++r) {
    std::vector<int> members;  // kept in ascending id
    double rload = 0.0;
    while (static_cast<int>(members.size()) < cap) {
      bool any_fit = false;
      for (int e = 0; e < E; ++e)
        if (expert_rank[e] < 0 && rload + static_cast<double>(load[e]) <= limit) any_fit = true;
      int best = -1;
      double best_aff = 0.0;
      for (int e = 0; e < E; ++e) {  // ascending id: ties keep the lower id
        if (expert_rank[e] >= 0) continue;
        if (any_fit && !(rload + static_cast<double>(load[e]) <= limit)) continue;
        double aff = 0.0;
        for (int f : members) aff += C(e, f);
        if (best < 0 || aff > best_aff || (aff == best_aff && total[e] > total[best])) {
          best = e;
          best_aff = aff;
        }
      }
      expert_rank[best] = r;
      members.insert(std::upper_bound(members.begin(), members.end(), best), best);
      rload += static_cast<double>(load[best]);
    }
  }
  return MOE_OK;
}
