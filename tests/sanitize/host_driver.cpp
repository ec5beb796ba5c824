// Drives the library's host-only code (csrc/host.cpp: geometry validation,
// static sizing, scratch layouts, the EPLB replica planner, status strings)
// for a build under AddressSanitizer and UndefinedBehaviorSanitizer.
// Exit status 0 = clean.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "moe_route_topk.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { std::printf("FAIL %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

int main() {
  // the workloads' geometries and their sizes
  const moe_geom_t shapes[] = {
      {16, 64, 8, 8, 2, 4, 2, 4, 4, 0, 0, 0},
      {96, 7168, 256, 256, 8, 256, 1, 1, 96, 0, 0, 0},
      {12288, 7168, 256, 256, 8, 128, 2, 128, 96, 0, 0, 0},
      {4096, 7168, 256, 288, 8, 288, 1, 1, 4096, 0, 0, 0},
      {46080, 7168, 256, 288, 8, 288, 1, 160, 288, 0, 160, 0},
      {0, 7168, 256, 256, 8, 128, 2, 128, 0, 0, 0, 0},
  };
  for (const moe_geom_t &g : shapes) {
    moe_sizes_t s;
    EXPECT(moe_plan_sizes(&g, 2048, &s) == MOE_OK);
    EXPECT(s.dispatch_bytes == (int64_t)g.D * s.dispatch_bytes_per_partition);
    EXPECT(moe_plan_sizes(&g, 0, &s) == MOE_OK);
  }
  // random geometries, valid or not: every call returns a status, nothing faults
  std::mt19937 rng(7);
  auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int ok = 0;
  for (int i = 0; i < 20000; ++i) {
    moe_geom_t g{};
    g.S = pick(0, 300);
    g.LB = pick(-2, 5000);
    g.T = pick(0, 3) == 0 ? pick(-5, 100000) : g.S * g.LB;
    g.H = 16 * pick(-1, 1100);
    g.E = pick(-1, 1100);
    g.P = g.E + pick(-2, 40);
    g.k = pick(-1, 20);
    g.D = pick(-1, 1100);
    g.Epp = pick(-1, 9);
    g.msg_bytes = pick(0, 3) == 0 ? 16 * pick(0, 1200) : 0;
    g.relays = pick(0, 4) == 0 ? pick(0, 300) : 0;
    g.reserved = pick(0, 50) == 0;
    moe_sizes_t s;
    const int st = moe_plan_sizes(&g, 64 * pick(-1, 300), &s);
    EXPECT(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED);
    ok += st == MOE_OK;
  }
  EXPECT(ok > 0);
  EXPECT(moe_plan_sizes(nullptr, 0, nullptr) == MOE_ERR_INVALID_ARG);
  // the replica planner on random counts, and the capacity error
  for (int trial = 0; trial < 200; ++trial) {
    const int E = pick(1, 64), budget = pick(0, 16), slices = pick(1, 6);
    const int D = E + budget;
    std::vector<int64_t> cnt((size_t)slices * E);
    for (auto &c : cnt) c = pick(0, 5000);
    std::vector<int32_t> prim(E), freec(D), ro(E + 1), rs(E + budget), sp(E + budget),
        sl(E + budget), sel(budget > 0 ? budget : 1);
    for (int e = 0; e < E; ++e) prim[e] = e;
    for (int d = 0; d < D; ++d) freec[d] = d >= E;
    EXPECT(moe_eplb_build_map(cnt.data(), slices, E, budget, D, prim.data(), freec.data(),
                              ro.data(), rs.data(), sp.data(), sl.data(), sel.data()) == MOE_OK);
    EXPECT(ro[E] == E + budget);
    if (budget > 0) {
      std::vector<int32_t> none(D, 0);
      EXPECT(moe_eplb_build_map(cnt.data(), slices, E, budget, D, prim.data(), none.data(),
                                ro.data(), rs.data(), sp.data(), sl.data(),
                                nullptr) == MOE_ERR_CAPACITY);
    }
  }
  for (int st = -6; st <= 0; ++st) EXPECT(moe_status_string(st) != nullptr);
  std::printf(fails ? "host driver FAILED\n" : "host driver ok\n");
  return fails ? 1 : 0;
}
