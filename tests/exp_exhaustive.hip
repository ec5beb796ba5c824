// The expert GEMM's SwiGLU epilogue takes e = fp32(exp(-(double)g)) with the
// device math library; the oracle takes the same expression with the host C
// library.  This program compares the two for every non-NaN fp32 input x (all
// 2^32 bit patterns, in chunks of 2^28): the GPU computes (float)exp((double)x)
// in a kernel compiled with the library's flags, the host recomputes it with
// its own exp, and every result must have the same bits.  Prints one line per
// chunk and a summary; exits 0 only when there is no mismatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

__global__ void exp_chunk(uint32_t base, uint32_t n, uint32_t *out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= n) return;
  const uint32_t b = base + i;
  float x;
  memcpy(&x, &b, 4);
  const float e = (float)exp((double)x);
  uint32_t r;
  memcpy(&r, &e, 4);
  out[i] = r;
}

int main() {
  const uint32_t chunk = 1u << 28;
  uint32_t *d = nullptr;
  if (hipMalloc(&d, (size_t)chunk * 4) != hipSuccess) return 2;
  std::vector<uint32_t> h(chunk);
  uint64_t mismatches = 0, nans = 0;
  for (uint64_t base = 0; base < (1ull << 32); base += chunk) {
    hipLaunchKernelGGL(exp_chunk, dim3(chunk / 256), dim3(256), 0, 0, (uint32_t)base, chunk, d);
    if (hipMemcpy(h.data(), d, (size_t)chunk * 4, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    uint64_t m = 0, nn = 0;
#pragma omp parallel for reduction(+ : m, nn) schedule(static)
    for (int64_t i = 0; i < (int64_t)chunk; ++i) {
      const uint32_t b = (uint32_t)(base + i);
      float x;
      memcpy(&x, &b, 4);
      if (std::isnan(x)) {
        ++nn;
        continue;
      }
      const float e = (float)exp((double)x);
      uint32_t r;
      memcpy(&r, &e, 4);
      if (r != h[i]) {
        ++m;
        if (m <= 3) printf("  mismatch x=%a host=%08x device=%08x\n", x, r, h[i]);
      }
    }
    mismatches += m;
    nans += nn;
    printf("chunk %08llx mismatches %llu\n", (unsigned long long)base, (unsigned long long)m);
    fflush(stdout);
  }
  printf("inputs %llu mismatches %llu\n", (unsigned long long)((1ull << 32) - nans),
         (unsigned long long)mismatches);
  (void)hipFree(d);
  return mismatches ? 1 : 0;
}
