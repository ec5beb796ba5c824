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
// Two fp32 values -> packed bf16 bits (lo in the low half), round to nearest
// even, by one v_cvt_pk_bf16_f32.  For every non-NaN fp32 input this gives the
// bits of the textbook rounding (u + 0x7fff + ((u >> 16) & 1)) >> 16, finite
// values that round past the largest bf16 becoming infinities (all 2^32
// inputs compared on the device); NaN inputs come out as quiet NaNs.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector((f2){lo, hi}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace moe
