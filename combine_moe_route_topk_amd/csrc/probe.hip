// Measurement support, not part of the MoE path: the int8 MFMA rate this
// device sustains, the ceiling the expert GEMMs are compared with next to the
// published 5.0 POP/s (which assumes the 2.4 GHz peak clock; the clock falls
// under a sustained MFMA load).  Every wavefront runs four independent chains
// of v_mfma_i32_32x32x32_i8 on register operands, so nothing but the matrix
// pipes and the clock bound it.
#include "common.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_i8_probe_kernel(int iters, int32_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, 3 * lane + 1, 5 * lane + 2, 7 * lane + 3};
  const v4i b = {lane + 11, 13 * lane, 17 * lane + 5, 19 * lane + 7};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace moe

extern "C" int moe_probe_mfma_i8(int32_t blocks, int32_t iters, int32_t *out, void *stream) {
  if (blocks <= 0 || iters <= 0 || !out) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(moe::mfma_i8_probe_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, iters, out);
  return moe::launch_status();
}
