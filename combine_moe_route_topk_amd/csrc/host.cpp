// Host-only parts of the C ABI (plain C++, no HIP): geometry validation, static
// sizing, scratch layouts, the EPLB replica planner and status strings.
#include <algorithm>
#include <cmath>
#include <limits>
#include <vector>

#include "sizes.h"

namespace moe {

int validate_geom(const moe_geom_t *g) {
  if (!g) return MOE_ERR_INVALID_ARG;
  if (g->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (g->T < 0 || g->H <= 0 || g->E <= 0 || g->P <= 0 || g->k <= 0 || g->D <= 0 || g->Epp <= 0 ||
      g->S <= 0 || g->LB < 0 || g->relays < 0)
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)g->S * g->LB != g->T) return MOE_ERR_INVALID_ARG;
  if (g->k > g->E || g->E > g->P) return MOE_ERR_INVALID_ARG;
  if (g->H % 16 != 0 || g->H > MOE_MAX_H) return MOE_ERR_UNSUPPORTED;
  if (g->k > MOE_MAX_K || g->E > MOE_MAX_E || g->P > MOE_MAX_P || g->D > MOE_MAX_D)
    return MOE_ERR_UNSUPPORTED;
  if (g->msg_bytes != 0 && (g->msg_bytes < g->H + 16 || g->msg_bytes % 16 != 0))
    return MOE_ERR_INVALID_ARG;
  if (g->relays >= g->D) return MOE_ERR_INVALID_ARG;
  // every row index must fit an int32
  int64_t rows = (int64_t)g->D * g->S * cap_of(*g);
  if (rows > INT32_MAX || (int64_t)g->T * g->k * 2 > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int64_t up256(int64_t x) { return (x + 255) / 256 * 256; }

DispatchScratch dispatch_scratch_layout(const moe_geom_t &g) {
  DispatchScratch L{};
  int64_t nc = (int64_t)g.S * chunks_per_source(g);
  int64_t o = 0;
  L.status = o;
  o += 256;
  L.hist_d = o;
  o = up256(o + 4 * (int64_t)g.D * (nc + 1));
  L.hist_p = o;
  o = up256(o + 4 * (int64_t)g.P * (nc + 1));
  L.route_rank = o;
  o = up256(o + 4 * (int64_t)g.T * g.k);
  L.slot_local = o;
  o = up256(o + 4 * (int64_t)g.P);
  L.total = o;
  return L;
}

FfnScratch ffn_scratch_layout(const moe_geom_t &g, int32_t I) {
  FfnScratch L{};
  int64_t rows = (int64_t)g.T * g.k;
  int64_t o = 0;
  L.tiles = o;
  o = up256(o + 4 * ((int64_t)g.P + 2));
  L.slot_of = o;
  o = up256(o + 4 * ffn_mtile_bound(g));
  L.pmax = o;
  o = up256(o + 4 * rows * (I / 64));
  L.h = o;
  o = up256(o + 4 * rows * I);
  L.hq = o;
  o = up256(o + rows * I);
  L.hs = o;
  o = up256(o + 4 * rows);
  L.total = o;
  return L;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_plan_sizes(const moe_geom_t *g, int32_t I, moe_sizes_t *out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (I < 0 || I % 64 != 0 || I > 16384) return MOE_ERR_UNSUPPORTED;
  const int64_t msg = msg_bytes_of(*g), cap = cap_of(*g);
  out->msg_bytes = msg;
  out->cap_rows = cap;
  out->dispatch_bytes_per_partition = (int64_t)g->S * cap * msg;
  out->dispatch_bytes = (int64_t)g->D * out->dispatch_bytes_per_partition;
  out->combine_bytes_per_partition = (int64_t)g->D * cap * g->H * 2;
  out->relay_bytes = g->relays ? (int64_t)(g->D - g->relays) * g->S * cap * msg : 0;
  out->return_bytes = (int64_t)g->T * g->k * g->H * 2 * (g->relays ? 2 : 1);
  out->router_scratch_bytes = router_scratch_bytes_of(*g);
  out->ret_q8_row_bytes = ret_q8_row_bytes_of(*g);
  out->ret_q8_bytes = (int64_t)g->T * g->k * out->ret_q8_row_bytes;
  out->dispatch_scratch_bytes = dispatch_scratch_layout(*g).total;
  out->ffn_scratch_bytes = I ? ffn_scratch_layout(*g, I).total : 0;
  const bool ffn = I > 0 && g->H % 128 == 0;
  out->w_gateup_packed_bytes = ffn ? packed_weight_bytes(MOE_PROJ_GATEUP, g->E, g->H, I) : 0;
  out->w_down_packed_bytes = ffn ? packed_weight_bytes(MOE_PROJ_DOWN, g->E, g->H, I) : 0;
  return MOE_OK;
}

// Replica selection and placement; see the header for the rules.
extern "C" int moe_eplb_build_map(const int64_t *token_count, int32_t slices, int32_t E,
                                  int32_t budget, int32_t D, const int32_t *primary_partition,
                                  const int32_t *free_slots, int32_t *replica_offsets,
                                  int32_t *replica_slots, int32_t *slot_partition,
                                  int32_t *slot_logical, int32_t *selected) {
  if (!token_count || !primary_partition || !free_slots || !replica_offsets || !replica_slots ||
      !slot_partition || !slot_logical)
    return MOE_ERR_INVALID_ARG;
  if (slices <= 0 || E <= 0 || budget < 0 || D <= 0 || E > MOE_MAX_E || E + budget > MOE_MAX_P)
    return MOE_ERR_INVALID_ARG;
  for (int e = 0; e < E; ++e)
    if (primary_partition[e] < 0 || primary_partition[e] >= D) return MOE_ERR_INVALID_ARG;

  std::vector<int> copies(E, 1);
  auto load = [&](int t, int e, int extra) {
    return (double)token_count[(int64_t)t * E + e] / (double)(copies[e] + extra);
  };
  // hottest expert of slice t under the current copies (lower id on ties)
  auto hottest = [&](int t) {
    int h = 0;
    for (int e = 1; e < E; ++e)
      if (load(t, e, 0) > load(t, h, 0)) h = e;
    return h;
  };
  std::vector<int> picks;
  for (int round = 0; round < budget; ++round) {
    std::vector<char> is_cand(E, 0);
    for (int t = 0; t < slices; ++t) is_cand[hottest(t)] = 1;
    int best = -1;
    double best_tail = std::numeric_limits<double>::infinity();
    for (int c = 0; c < E; ++c) {
      if (!is_cand[c]) continue;
      double tail = 0.0;
      for (int t = 0; t < slices; ++t) {
        double m = 0.0;
        for (int e = 0; e < E; ++e) m = std::max(m, load(t, e, e == c));
        tail += m;
      }
      if (tail < best_tail) {
        best_tail = tail;
        best = c;
      }
    }
    if (best < 0) break;
    copies[best] += 1;
    picks.push_back(best);
  }

  std::vector<double> total(E, 0.0), pload(D, 0.0);
  for (int t = 0; t < slices; ++t)
    for (int e = 0; e < E; ++e) total[e] += (double)token_count[(int64_t)t * E + e];
  for (int e = 0; e < E; ++e) {
    pload[primary_partition[e]] += total[e] / copies[e];
    slot_partition[e] = primary_partition[e];
    slot_logical[e] = e;
  }
  std::vector<int> order(picks);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return total[a] > total[b]; });
  std::vector<int> freec(free_slots, free_slots + D);
  for (size_t i = 0; i < order.size(); ++i) {
    int e = order[i], target = -1;
    for (int d = 0; d < D; ++d)
      if (freec[d] > 0 && (target < 0 || pload[d] < pload[target])) target = d;
    if (target < 0) return MOE_ERR_CAPACITY;
    pload[target] += total[e] / copies[e];
    freec[target] -= 1;
    slot_partition[E + i] = target;
    slot_logical[E + i] = e;
  }
  const int P = E + budget;
  for (int p = E + (int)order.size(); p < P; ++p) slot_partition[p] = slot_logical[p] = -1;
  // replica lists: slots of each expert in ascending slot id
  std::vector<std::vector<int>> lists(E);
  for (int p = 0; p < P; ++p)
    if (slot_logical[p] >= 0) lists[slot_logical[p]].push_back(p);
  int n = 0;
  for (int e = 0; e < E; ++e) {
    replica_offsets[e] = n;
    for (int p : lists[e]) replica_slots[n++] = p;
  }
  replica_offsets[E] = n;
  if (selected)
    for (size_t i = 0; i < picks.size(); ++i) selected[i] = picks[i];
  return MOE_OK;
}

extern "C" const char *moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported geometry";
    case MOE_ERR_CAPACITY: return "capacity exceeded";
    case MOE_ERR_STALE: return "stale event (metadata or messages of another dispatch)";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}
