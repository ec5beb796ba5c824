// Internal helpers of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_route_topk.h"
#include "sizes.h"

namespace moe {

// Gate logits into out (router.hip): [T][E] when router_splits(g) == 1, else
// the partial sums [splits][T][E]; and the host checks shared by the two gate
// entry points.
int router_partials(const void *x, const void *w_router, const moe_geom_t &g, float *out,
                    hipStream_t s);
int router_check(const void *x, const void *w_router, const moe_geom_t *g, void *scratch,
                 size_t scratch_bytes);
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
inline int launch_status() { return hip_status(hipGetLastError()); }

// ---------------------------------------------------------- device side ---

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
// round to nearest even (finite inputs; infinities stay infinite, NaN is kept
// a NaN); written without branches so that it vectorizes in epilogues
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t special = (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u & 0x7f800000u) == 0x7f800000u ? special : rounded;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace moe
