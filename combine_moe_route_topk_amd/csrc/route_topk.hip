// Gate top-k + EPLB replica gather + per-expert collect histogram.
//
// [XDS 合设 A2A, P038; CMI EP320 gate.topk; XDS 专家负载均衡 P068 (collect),
//  P078-P079 / Fig. 12 (logical -> physical gather, round robin by position)]
//
// One 64-lane wavefront per token: lane l holds the scores of experts
// l*EPL .. l*EPL+EPL-1 as 32-bit order keys (unsigned order = float order).
// The k-th largest key is found by a radix select over its 32 bits, one bit
// per round, where each round's count is the popcount of the wavefront's
// ballots: scalar work, no cross-lane data movement.  The select stops as soon
// as exactly k keys reach the threshold; otherwise the threshold is the k-th
// largest key itself and the keys equal to it are taken lowest expert id
// first.  The k chosen keys are then read out with readlane into lanes
// 0..k-1, each lane counting the chosen keys that outrank its own (score
// descending, id ascending), so lane j ends up knowing its route's rank.
#include "common.h"

namespace moe {
namespace {

constexpr int kBlock = 1024;      // threads per block (16 wavefronts)
constexpr int kMaxBlocks = 256;   // one block per CU: bounds the histogram's global atomics

__device__ __forceinline__ uint32_t order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 are the same score
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ int lowest_lane(uint64_t m) { return __builtin_ctzll(m); }

__global__ void zero_i32(int32_t *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Loads the EPL raw logits of one lane (FULL: E == 64*EPL, so the lane's
// run is whole and aligned to its size and can go as one vector load).
// fp32 logits may come as nsplit partial sums split_stride floats apart (the
// gate GEMM's K splits), added in split order: the same fp32 sums as the
// gate's own reduction, so the logits are the same bits.
template <int EPL, bool BF16, bool FULL>
__device__ __forceinline__ void load_row(const void *logits, int64_t t, int E, int lane,
                                         int nsplit, int64_t split_stride, float (&v)[EPL]) {
  if constexpr (BF16) {
    const uint16_t *row = (const uint16_t *)logits + t * E + lane * EPL;
    if constexpr (FULL) {
      constexpr int kAlign = EPL * 2 >= 16 ? 16 : EPL * 2;
      const uint16_t *p = (const uint16_t *)__builtin_assume_aligned(row, kAlign);
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i] = bf16_bits_to_f32(__builtin_nontemporal_load(p + i));
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        v[i] = lane * EPL + i < E ? bf16_bits_to_f32(__builtin_nontemporal_load(row + i)) : 0.0f;
    }
  } else {
    const float *row = (const float *)logits + t * E + lane * EPL;
    for (int sp = 0; sp < nsplit; ++sp, row += split_stride) {
      float u[EPL];
      if constexpr (FULL) {
        constexpr int kAlign = EPL * 4 >= 16 ? 16 : EPL * 4;
        const float *p = (const float *)__builtin_assume_aligned(row, kAlign);
#pragma unroll
        for (int i = 0; i < EPL; ++i) u[i] = __builtin_nontemporal_load(p + i);
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          u[i] = lane * EPL + i < E ? __builtin_nontemporal_load(row + i) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i] = sp == 0 ? u[i] : v[i] + u[i];
    }
  }
}

template <int EPL, bool BF16, bool FULL>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(
    const void *__restrict__ logits, const float *__restrict__ bias, int gating,
    const int32_t *__restrict__ roff, const int32_t *__restrict__ rslots, int T, int E, int P,
    int k, int LB, int nsplit, int64_t split_stride, float *__restrict__ logits_out,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ phys_ids,
    int32_t *__restrict__ expert_counts) {
  extern __shared__ int32_t hist[];  // [E] when expert_counts != nullptr
  const int lane = threadIdx.x & 63;
  if (expert_counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
  }
  float bv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    bv[i] = bias && e < E ? bias[e] : 0.0f;
  }
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  // the wavefront index is uniform; saying so keeps the token loop and the
  // select below on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  float raw[EPL];
  if (t < T) load_row<EPL, BF16, FULL>(logits, t, E, lane, nsplit, split_stride, raw);
  for (; t < T; t += nwaves) {
    if (logits_out) {  // the summed logits, for callers that keep them
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane * EPL + i < E) logits_out[t * E + lane * EPL + i] = raw[i];
    }
    uint32_t ord[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) ord[i] = lane * EPL + i < E ? order_key(raw[i] + bv[i]) : 0u;
    if (t + nwaves < T) load_row<EPL, BF16, FULL>(logits, t + nwaves, E, lane, nsplit, split_stride, raw);

    // radix select of the k-th largest key (invalid lanes hold 0, below every
    // candidate, and lose every tie on id)
    uint32_t tau = 0;
    int b = 31, c;
    do {
      const uint32_t cand = tau | (1u << b);
      c = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) c += popc64(__ballot(ord[i] >= cand));
      if (c >= k) tau = cand;
      --b;
    } while (b >= 0 && c != k);
    const bool exact = c == k;
    uint64_t sel[EPL];
    if (exact) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) sel[i] = __ballot(ord[i] >= tau);
    } else {
      // keys above tau are all chosen; the rest come from the keys equal to
      // tau in ascending expert id (lane-major, then i)
      uint64_t eq[EPL];
      int need = k;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        sel[i] = __ballot(ord[i] > tau);
        eq[i] = __ballot(ord[i] == tau);
        need -= popc64(sel[i]);
      }
      for (; need > 0; --need) {
        int best = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (eq[i]) best = min(best, lowest_lane(eq[i]) * EPL + i);
        const int bl = best / EPL, bi = best % EPL;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (i == bi) {
            eq[i] &= ~(1ull << bl);
            sel[i] |= 1ull << bl;
          }
      }
    }

    // read the k chosen keys out into lanes 0..k-1 and rank them
    uint32_t my_o = 0;
    int my_e = 0, rank = 0, j = 0;  // j: keys read out so far
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      uint64_t m = sel[i];
      while (m) {
        const int l = lowest_lane(m);
        m &= m - 1;
        const uint32_t O = (uint32_t)__builtin_amdgcn_readlane((int)ord[i], l);
        const int Ei = l * EPL + i;
        const bool older = lane < j;
        const bool beats = older & ((O > my_o) | ((O == my_o) & (Ei < my_e)));
        const uint64_t above = __ballot(older & !beats);
        rank += beats ? 1 : 0;
        if (lane == j) {
          my_o = O;
          my_e = Ei;
          rank = popc64(above);
        }
        ++j;
      }
    }

    // lane l < k holds the route of rank `rank`
    const bool act = lane < k;
    const float s = key_score(my_o);
    const int l0 = lowest_lane(__ballot(act && rank == 0));
    const float s0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(s), l0));
    float a = 0.0f;
    if (act) a = gating == MOE_GATING_SOFTMAX ? expf(s - s0) : 1.0f / (1.0f + expf(-s));
    float sum = a;
    for (int o = 1; o < k; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (act) {
      const int64_t o = t * k + rank;
      topk_ids[o] = my_e;
      topk_w[o] = a / sum;
      int p = my_e;
      if (roff) {
        const int r0 = roff[my_e], n = roff[my_e + 1] - r0;
        p = -1;
        if (n > 0 && r0 >= 0 && r0 + n <= P) {
          const int b = (int)(t % LB);
          p = rslots[r0 + b % n];
          if (p < 0 || p >= P) p = -1;
        }
      }
      phys_ids[o] = p;
      if (expert_counts) atomicAdd(&hist[my_e], 1);
    }
  }
  if (expert_counts) {
    __syncthreads();
    // Two counters per 64-bit add when the pair is 8-byte aligned: each
    // counter's total is at most T < 2^31, so the low half never carries.
    if ((E & 1) == 0 && ((uintptr_t)expert_counts & 7) == 0) {
      unsigned long long *c2 = (unsigned long long *)expert_counts;
      for (int e = threadIdx.x; e < E / 2; e += blockDim.x) {
        const unsigned long long v =
            (unsigned long long)(uint32_t)hist[2 * e] | ((unsigned long long)(uint32_t)hist[2 * e + 1] << 32);
        if (v) atomicAdd(c2 + e, v);
      }
    } else {
      for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (hist[e]) atomicAdd(&expert_counts[e], hist[e]);
    }
  }
}

struct RouteIn {  // the logits: one array, or nsplit partial sums split_stride apart
  const void *logits;
  int nsplit;
  int64_t split_stride;
  float *logits_out;  // the summed logits are written here when not null
};

template <int EPL, bool BF16, bool FULL>
hipError_t launch_route3(const RouteIn &in, const float *bias, int gating, const int32_t *roff,
                         const int32_t *rslots, const moe_geom_t &g, int32_t *ids, float *w,
                         int32_t *phys, int32_t *counts, hipStream_t st) {
  const int waves = kBlock / 64;
  const int blocks = (int)std::min<int64_t>(((int64_t)g.T + waves - 1) / waves, kMaxBlocks);
  const size_t lds = counts ? sizeof(int32_t) * g.E : 0;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((route_topk_kernel<EPL, BF16, FULL>), dim3(blocks), dim3(kBlock), lds, st,
                     in.logits, bias, gating, roff, rslots, g.T, g.E, g.P, g.k, g.LB, in.nsplit,
                     in.split_stride, in.logits_out, ids, w, phys, counts);
  return hipGetLastError();
}

template <int EPL>
hipError_t launch_route(const RouteIn &in, bool bf16, const float *bias, int gating,
                        const int32_t *roff, const int32_t *rslots, const moe_geom_t &g,
                        int32_t *ids, float *w, int32_t *phys, int32_t *counts, hipStream_t st) {
  const bool full = g.E == 64 * EPL;
  if (bf16)
    return full ? launch_route3<EPL, true, true>(in, bias, gating, roff, rslots, g, ids, w, phys,
                                                 counts, st)
                : launch_route3<EPL, true, false>(in, bias, gating, roff, rslots, g, ids, w, phys,
                                                  counts, st);
  return full ? launch_route3<EPL, false, true>(in, bias, gating, roff, rslots, g, ids, w, phys,
                                                counts, st)
              : launch_route3<EPL, false, false>(in, bias, gating, roff, rslots, g, ids, w, phys,
                                                 counts, st);
}

// Checks shared by the two top-k entry points (no launch on error).
int route_check(moe_gating_t gating, const int32_t *roff, const int32_t *rslots,
                const moe_geom_t *g, int32_t *topk_ids, float *topk_w, int32_t *phys_ids) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (g->T > 0 && (!topk_ids || !topk_w || !phys_ids)) return MOE_ERR_INVALID_ARG;
  if (gating != MOE_GATING_SOFTMAX && gating != MOE_GATING_SIGMOID) return MOE_ERR_INVALID_ARG;
  if ((roff == nullptr) != (rslots == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!roff && g->P != g->E) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int route_run(const RouteIn &in, bool bf16, const float *bias, moe_gating_t gating,
              const int32_t *roff, const int32_t *rslots, const moe_geom_t *g, int32_t *topk_ids,
              float *topk_w, int32_t *phys_ids, int32_t *expert_counts, hipStream_t s) {
  int st;
  if (expert_counts) {
    hipLaunchKernelGGL(zero_i32, dim3((g->E + 255) / 256), dim3(256), 0, s, expert_counts, g->E);
    if ((st = launch_status()) != MOE_OK) return st;
  }
  hipError_t e;
  const int E = g->E;
  if (E <= 64)
    e = launch_route<1>(in, bf16, bias, gating, roff, rslots, *g, topk_ids, topk_w, phys_ids,
                        expert_counts, s);
  else if (E <= 128)
    e = launch_route<2>(in, bf16, bias, gating, roff, rslots, *g, topk_ids, topk_w, phys_ids,
                        expert_counts, s);
  else if (E <= 256)
    e = launch_route<4>(in, bf16, bias, gating, roff, rslots, *g, topk_ids, topk_w, phys_ids,
                        expert_counts, s);
  else if (E <= 512)
    e = launch_route<8>(in, bf16, bias, gating, roff, rslots, *g, topk_ids, topk_w, phys_ids,
                        expert_counts, s);
  else
    e = launch_route<16>(in, bf16, bias, gating, roff, rslots, *g, topk_ids, topk_w, phys_ids,
                         expert_counts, s);
  return hip_status(e);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_route_topk(const void *logits, moe_dtype_t logits_dtype, const float *bias,
                              moe_gating_t gating, const int32_t *replica_offsets,
                              const int32_t *replica_slots, const moe_geom_t *g, int32_t *topk_ids,
                              float *topk_w, int32_t *phys_ids, int32_t *expert_counts,
                              void *stream) {
  int st = route_check(gating, replica_offsets, replica_slots, g, topk_ids, topk_w, phys_ids);
  if (st != MOE_OK) return st;
  if (g->T > 0 && !logits) return MOE_ERR_INVALID_ARG;
  if (logits_dtype != MOE_DTYPE_F32 && logits_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  const RouteIn in{logits, 1, 0, nullptr};
  return route_run(in, logits_dtype == MOE_DTYPE_BF16, bias, gating, replica_offsets,
                   replica_slots, g, topk_ids, topk_w, phys_ids, expert_counts,
                   (hipStream_t)stream);
}

extern "C" int moe_router_topk(const void *x, const void *w_router, const float *bias,
                               moe_gating_t gating, const int32_t *replica_offsets,
                               const int32_t *replica_slots, const moe_geom_t *g, float *logits,
                               int32_t *topk_ids, float *topk_w, int32_t *phys_ids,
                               int32_t *expert_counts, void *scratch, size_t scratch_bytes,
                               void *stream) {
  int st = route_check(gating, replica_offsets, replica_slots, g, topk_ids, topk_w, phys_ids);
  if (st != MOE_OK) return st;
  if ((st = router_check(x, w_router, g, scratch, scratch_bytes)) != MOE_OK || g->T == 0) return st;
  if (logits && !aligned16(logits)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // one split: the gate writes the logits themselves (the caller's, or scratch)
  // and the top-k reads them; several: the top-k adds the partial sums
  const int ks = router_splits(*g);
  float *part = ks == 1 && logits ? logits : (float *)scratch;
  if ((st = router_partials(x, w_router, *g, part, s)) != MOE_OK) return st;
  const RouteIn in{part, ks, (int64_t)g->T * g->E, ks == 1 ? nullptr : logits};
  return route_run(in, false, bias, gating, replica_offsets, replica_slots, g, topk_ids, topk_w,
                   phys_ids, expert_counts, s);
}
