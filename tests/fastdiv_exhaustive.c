/*
 * Exhaustive check of the division-free quotient used by the expert GEMM's
 * INT8-return epilogue (test infrastructure; no part of the library).
 *
 * For every positive finite bf16 amax and every bf16 y with |y| <= amax:
 *   s = amax / 127 (IEEE), and when s >= 2^-100:
 *   r = 1 / s (IEEE), q0 = y * r, e = fma(-q0, s, y), q = fma(e, r, q0);
 *   otherwise q = y / s.
 * The INT8 code clamp(rint(q), +-127) must equal the code of the IEEE quotient
 * y / s.  Prints the counts and exits non-zero on any mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static int code(float q) { return (int)fminf(fmaxf(rintf(q), -127.0f), 127.0f); }

int main(void) {
  const float threshold = 0x1p-100f;
  long long pairs = 0, fast = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, fast, bad)
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf16(ab);
    const float s = amax / 127.0f;
    const int use_fast = s >= threshold;
    const float r = 1.0f / s;
    for (uint32_t yb = 0; yb < 0x10000; ++yb) {
      const float y = bf16(yb);
      if (!(fabsf(y) <= amax)) continue;
      ++pairs;
      float q = y / s;
      const int want = code(q);
      if (use_fast) {
        ++fast;
        const float q0 = y * r;
        q = fmaf(fmaf(-q0, s, y), r, q0);
      }
      if (code(q) != want) ++bad;
    }
  }
  printf("pairs %lld fast %lld mismatches %lld\n", pairs, fast, bad);
  return bad != 0;
}
