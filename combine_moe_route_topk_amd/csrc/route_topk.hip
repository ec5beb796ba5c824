// Gate top-k + EPLB replica gather + per-expert collect histogram.
//
// [XDS 合设 A2A, P038; CMI EP320 gate.topk; XDS 专家负载均衡 P068 (collect),
//  P078-P079 / Fig. 12 (logical -> physical gather, round robin by position)]
//
// One 64-lane wavefront per token: lane l holds the scores of experts
// l*EPL .. l*EPL+EPL-1.  Each score is packed with its id into a 64-bit key
// that orders by (score descending, id ascending); k rounds of a wavefront
// max-reduction pick the routes in order, so ties resolve to the lower id
// exactly as a stable sort would, with no fp comparison subtleties.
#include "common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;          // wavefronts per block
constexpr int kTokensPerWave = 4;  // tokens each wavefront handles in turn

__device__ __forceinline__ uint64_t make_key(float s, int e) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 are the same score
  uint32_t u = __float_as_uint(s);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t ord = (uint32_t)(key >> 32);
  uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ void zero_i32(int32_t *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int EPL, bool BF16>
__global__ __launch_bounds__(64 * kWaves) void route_topk_kernel(
    const void *__restrict__ logits, const float *__restrict__ bias, int gating,
    const int32_t *__restrict__ roff, const int32_t *__restrict__ rslots, int T, int E, int P,
    int k, int LB, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ phys_ids, int32_t *__restrict__ expert_counts) {
  extern __shared__ int32_t hist[];  // [E] when expert_counts != nullptr
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (expert_counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
  }
  const int64_t t_base = ((int64_t)blockIdx.x * kWaves + wave) * kTokensPerWave;
  for (int it = 0; it < kTokensPerWave; ++it) {
    const int64_t t = t_base + it;
    if (t >= T) break;
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      key[i] = 0;  // below every real score key
      if (e < E) {
        float v = BF16 ? bf16_bits_to_f32(((const uint16_t *)logits)[t * E + e])
                       : ((const float *)logits)[t * E + e];
        float b = bias ? bias[e] : 0.0f;
        key[i] = make_key(v + b, e);
      }
    }
    uint64_t mine = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) m = key[i] > m ? key[i] : m;
      m = wave_max_u64(m);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (key[i] == m) key[i] = 0;
      if (lane == j) mine = m;
    }
    // lanes 0..k-1 now hold route j = lane
    const bool act = lane < k;
    const float s = key_score(mine);
    const float s0 = __shfl(s, 0, 64);
    float a = 0.0f;
    if (act) a = gating == MOE_GATING_SOFTMAX ? expf(s - s0) : 1.0f / (1.0f + expf(-s));
    const float sum = wave_sum_f32(a);
    if (act) {
      const int e = key_id(mine);
      const int64_t o = t * k + lane;
      topk_ids[o] = e;
      topk_w[o] = a / sum;
      int p = e;
      if (roff) {
        const int r0 = roff[e], n = roff[e + 1] - r0;
        p = -1;
        if (n > 0 && r0 >= 0 && r0 + n <= P) {
          const int b = (int)(t % LB);
          p = rslots[r0 + b % n];
          if (p < 0 || p >= P) p = -1;
        }
      }
      phys_ids[o] = p;
      if (expert_counts) atomicAdd(&hist[e], 1);
    }
  }
  if (expert_counts) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      if (hist[e]) atomicAdd(&expert_counts[e], hist[e]);
  }
}

template <int EPL>
hipError_t launch_route(const void *logits, bool bf16, const float *bias, int gating,
                        const int32_t *roff, const int32_t *rslots, const moe_geom_t &g,
                        int32_t *ids, float *w, int32_t *phys, int32_t *counts, hipStream_t st) {
  const int per_block = kWaves * kTokensPerWave;
  const int blocks = (g.T + per_block - 1) / per_block;
  const size_t lds = counts ? sizeof(int32_t) * g.E : 0;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL((route_topk_kernel<EPL, true>), dim3(blocks), dim3(64 * kWaves), lds, st,
                       logits, bias, gating, roff, rslots, g.T, g.E, g.P, g.k, g.LB, ids, w, phys,
                       counts);
  else
    hipLaunchKernelGGL((route_topk_kernel<EPL, false>), dim3(blocks), dim3(64 * kWaves), lds, st,
                       logits, bias, gating, roff, rslots, g.T, g.E, g.P, g.k, g.LB, ids, w, phys,
                       counts);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_route_topk(const void *logits, moe_dtype_t logits_dtype, const float *bias,
                              moe_gating_t gating, const int32_t *replica_offsets,
                              const int32_t *replica_slots, const moe_geom_t *g, int32_t *topk_ids,
                              float *topk_w, int32_t *phys_ids, int32_t *expert_counts,
                              void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (g->T > 0 && (!logits || !topk_ids || !topk_w || !phys_ids)) return MOE_ERR_INVALID_ARG;
  if (logits_dtype != MOE_DTYPE_F32 && logits_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (gating != MOE_GATING_SOFTMAX && gating != MOE_GATING_SIGMOID) return MOE_ERR_INVALID_ARG;
  if ((replica_offsets == nullptr) != (replica_slots == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!replica_offsets && g->P != g->E) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (expert_counts) {
    hipLaunchKernelGGL(zero_i32, dim3((g->E + 255) / 256), dim3(256), 0, s, expert_counts, g->E);
    if ((st = launch_status()) != MOE_OK) return st;
  }
  const bool bf16 = logits_dtype == MOE_DTYPE_BF16;
  hipError_t e;
  const int E = g->E;
  if (E <= 64)
    e = launch_route<1>(logits, bf16, bias, gating, replica_offsets, replica_slots, *g, topk_ids,
                        topk_w, phys_ids, expert_counts, s);
  else if (E <= 128)
    e = launch_route<2>(logits, bf16, bias, gating, replica_offsets, replica_slots, *g, topk_ids,
                        topk_w, phys_ids, expert_counts, s);
  else if (E <= 256)
    e = launch_route<4>(logits, bf16, bias, gating, replica_offsets, replica_slots, *g, topk_ids,
                        topk_w, phys_ids, expert_counts, s);
  else if (E <= 512)
    e = launch_route<8>(logits, bf16, bias, gating, replica_offsets, replica_slots, *g, topk_ids,
                        topk_w, phys_ids, expert_counts, s);
  else
    e = launch_route<16>(logits, bf16, bias, gating, replica_offsets, replica_slots, *g, topk_ids,
                         topk_w, phys_ids, expert_counts, s);
  return hip_status(e);
}
