/*
 * Exhaustive checks of the two division shortcuts used by libkvc's kernels
 * (kvc_kernels.hip: div_const; kvc_arch.h: recip_newton), evaluated here with the same
 * binary32 operations (C float with -ffp-contract=off, fmaf):
 *   1. RN(a / N) = q0 + e*r with r = RN(1/N), q0 = RN(a*r), e = fma(-q0, N, a),
 *      for every non-negative finite binary32 a and N in {7, 15, 127};
 *   2. RN(1/h) = y0 + e*y0 with e = fma(-h, y0, 1), for every positive finite
 *      FP16 value h and every start y0 within one ulp of 1/h (the hardware
 *      reciprocal estimate is accurate to 1 ulp).
 * The reference quotient is C's correctly rounded float division.
 * Prints one line per check: "<name> <mismatches> <cases>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t f_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

int main(void) {
  const int divisors[3] = {7, 15, 127};
  for (int t = 0; t < 3; t++) {
    const float n = (float)divisors[t];
    volatile float one = 1.0f;
    const float r = one / n;
    unsigned long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
    for (long i = 0; i < 0x7F800000L; i++) {
      const float a = bits_f((uint32_t)i);
      const float q0 = a * r;
      const float q = fmaf(fmaf(-q0, n, a), r, q0);
      if (f_bits(q) != f_bits(a / n)) bad++;
    }
    printf("div_const_%d %lu %ld\n", divisors[t], bad, 0x7F800000L);
  }
  unsigned long bad = 0, cases = 0;
  for (uint32_t h = 1; h < 0x7C00; h++) {
    const uint32_t e = h >> 10, m = h & 0x3FF;
    const float x = e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
    const float ref = 1.0f / x;
    for (int d = -1; d <= 1; d++) {
      const float y0 = bits_f(f_bits(ref) + (uint32_t)d);
      const float y = fmaf(fmaf(-x, y0, 1.0f), y0, y0);
      cases++;
      if (f_bits(y) != f_bits(ref)) bad++;
    }
  }
  printf("recip_f16 %lu %lu\n", bad, cases);
  return 0;
}
