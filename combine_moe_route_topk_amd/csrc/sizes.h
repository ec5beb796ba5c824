// Sizing and layout helpers of the C ABI shared by the host code and the
// kernels (plain C++: no HIP types, so the host code also builds with a host
// compiler, for example under the sanitizers).
#pragma once

#include <stdint.h>

#include "moe_route_topk.h"

namespace moe {

inline int64_t msg_bytes_of(const moe_geom_t &g) {
  return g.msg_bytes ? (int64_t)g.msg_bytes : (((int64_t)g.H + 16 + 127) / 128) * 128;
}
inline int64_t cap_of(const moe_geom_t &g) { return (int64_t)g.LB * (g.k < g.Epp ? g.k : g.Epp); }
// Router GEMM (bf16 [T][H] x [E][H]^T) tiles: 192 tokens x 256 experts, K
// steps of 64 elements.  K splits: the largest divisor of the step count that
// keeps tiles x splits <= 256 (one block per CU), at most 32; 0 = H not a
// multiple of 64.
constexpr int kRouterRows = 192, kRouterCols = 256, kRouterStep = 64;
inline int router_splits(const moe_geom_t &g) {
  if (g.H <= 0 || g.H % kRouterStep != 0) return 0;
  const int64_t tiles = ((int64_t)g.T + kRouterRows - 1) / kRouterRows *
                        ((g.E + kRouterCols - 1) / kRouterCols);
  const int steps = g.H / kRouterStep;
  int ks = 1;
  for (int d = 2; d <= 32 && d <= steps; ++d)
    if (steps % d == 0 && tiles * d <= 256) ks = d;
  return ks;
}
inline int64_t router_scratch_bytes_of(const moe_geom_t &g) {
  return (int64_t)router_splits(g) * g.T * g.E * 4;
}
// INT8 return row: H codes, then one fp32 scale per MOE_RET_Q8_BLOCK columns.
// Rows are whole 128-byte cache lines, so that every 256-column block of codes
// a GEMM tile stores covers whole lines (a row of H + 4 nblk bytes rounded only
// to 16 would leave most blocks straddling lines, written partially by two tiles)
inline int64_t ret_q8_row_bytes_of(const moe_geom_t &g) {
  const int64_t nblk = ((int64_t)g.H + MOE_RET_Q8_BLOCK - 1) / MOE_RET_Q8_BLOCK;
  return ((int64_t)g.H + 4 * nblk + 127) / 128 * 128;
}

// Rows of an expert-GEMM m-tile; a slot of n rows has ceil(n / 128) m-tiles,
// so T k routes make at most T k / 128 + P of them.
constexpr int kFfnTileRows = 128;
inline int64_t ffn_mtile_bound(const moe_geom_t &g) {
  return (int64_t)g.T * g.k / kFfnTileRows + g.P;
}

// Image of the INT8 expert weights (moe_pack_expert_weights): one 16 KB block
// per (expert, n-tile, 64-byte K step), n-tiles of 128 gate/up pairs
// (gate/up) or 256 output channels (down), K padded to whole groups of four
// steps.
constexpr int64_t kPackedStepBytes = 256 * 64;
constexpr int packed_ntiles(int proj, int H, int I) {
  return proj == MOE_PROJ_GATEUP ? (I + 127) / 128 : (H + 255) / 256;
}
constexpr int packed_ksteps(int K) { return (K / 64 + 3) & ~3; }
inline int64_t packed_weight_bytes(int proj, int E, int H, int I) {
  const int K = proj == MOE_PROJ_GATEUP ? H : I;
  return (int64_t)E * packed_ntiles(proj, H, I) * packed_ksteps(K) * kPackedStepBytes;
}

// Routes per dispatch chunk: chunks never straddle a source partition.
constexpr int kChunkRoutes = 256;
inline int chunk_tokens(const moe_geom_t &g) {
  int ct = kChunkRoutes / g.k;
  ct = ct < g.LB ? ct : g.LB;
  return ct > 0 ? ct : 1;
}
inline int64_t chunks_per_source(const moe_geom_t &g) {
  int ct = chunk_tokens(g);
  return ((int64_t)g.LB + ct - 1) / ct;
}

int validate_geom(const moe_geom_t *g);

// Byte layout of the dispatch scratch (all offsets 256-aligned).
struct DispatchScratch {
  int64_t status;       // int32 device status word (then one unused int32)
  int64_t hist_d;       // int32 [D][NC+1]  per-chunk route counts per destination partition
  int64_t hist_p;       // int32 [P][NC+1]  per-chunk route counts per slot
  int64_t route_rank;   // int32 [T*k]    (rank in chunk for d) | (rank in chunk for p) << 16
  int64_t slot_local;   // int32 [P]
  int64_t total;
};
DispatchScratch dispatch_scratch_layout(const moe_geom_t &g);

// Byte layout of the expert-FFN scratch.
struct FfnScratch {
  int64_t tiles;     // int32 [P + 1]: exclusive prefix of per-slot m-tile counts, then the total
  int64_t slot_of;   // int32 [T*k/128 + P]: the slot of each m-tile (slot-major order)
  int64_t pmax;      // fp32 [I/128][T*k] max |h| of each row over each gate-up n-tile, n-tile
                     // major (a GEMM block stores its rows' maxima as one run); I/64 per row
                     // reserved
  int64_t h;         // fp32 [T*k][I]
  int64_t hq;        // int8 [T*k][I]
  int64_t hs;        // fp32 [T*k]
  int64_t total;
};
FfnScratch ffn_scratch_layout(const moe_geom_t &g, int32_t I);

}  // namespace moe
