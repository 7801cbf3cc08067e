/*
 * Exhaustive check of the uniform-codec quotient in libkvc's encode kernel
 * (kvc_kernels.hip: uniform_code), evaluated with the same binary32
 * operations (C float with -ffp-contract=off, fmaf).  The defined code is
 *     code = clamp(RNE(RN(d / s)), 0, top),  d = RN(x - m_h), s = sigma_h,
 * with s a positive finite FP16 value and top = 2^b - 1 (7 or 15).  The
 * kernel forms the quotient from y = RN(1/s) (recip_newton, checked
 * separately):
 *     q0 = RN(d*y), q = RN(q0 + RN(d - q0*s)*y)   (two FMAs),
 * and the code from the bits of RN(q + 1.5*2^23), clamped as integers.
 *
 * 1. "pairs": q == RN(d/s) for every binary32 significand of d in [1, 2) and
 *    every FP16 significand of s in [1, 2) (2^33 pairs).  Scaling d or s by
 *    a power of two scales q0, q and RN(d/s) by the same power while every
 *    intermediate stays normal and the residual d - q0*s stays exact, which
 *    holds whenever d >= s/4 and d/s < 2^100 (the residual is a multiple of
 *    ulp(q0)*ulp(s) > 2^-149 below ulp(d)); so q == RN(d/s) for every such
 *    d and every positive finite FP16 s, normal or subnormal (a subnormal
 *    FP16 value is a binary32 normal with one of the same significands).
 *    For 0 <= d < s/4 both codes are 0: RN(d/s) <= 1/4 and q < 1/2.
 * 2. "ties": the whole code pipeline against the definition, for every
 *    positive finite FP16 s, every k < top and the 2049 binary32 values d
 *    closest to (k + 1/2)*s, and for d at and around top*s (the clamp).
 * 3. "small": both codes are 0 for every binary32 d in [0, s/4] with s the
 *    smallest FP16 subnormal, normal and the largest FP16 value, d ranging
 *    over all subnormal binary32 values and 2^20 values below s/4.
 * Prints one line per check: "<name> <mismatches> <cases>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t f_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

static float f16_value(uint32_t h) {
  const uint32_t e = (h >> 10) & 31, m = h & 0x3FF;
  return e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
}

#define MAGIC 0x4B400000
static int kernel_code(float d, float s, float y, int top) {
  const float q0 = d * y;
  const float q = fmaf(fmaf(-q0, s, d), y, q0);
  int t = (int)f_bits(q + 12582912.0f);
  t = t < MAGIC ? MAGIC : (t > MAGIC + top ? MAGIC + top : t);
  return t - MAGIC;
}
static int defined_code(float d, float s, int top) {
  const float c = rintf(d / s);
  return c < 0.0f ? 0 : (c > (float)top ? top : (int)c);
}

int main(void) {
  volatile float one = 1.0f;
  {
    unsigned long bad = 0, cases = 0;
#pragma omp parallel for reduction(+ : bad, cases) schedule(dynamic, 1)
    for (int m = 0; m < 1024; m++) {
      const float s = 1.0f + (float)m / 1024.0f;
      const float y = one / s;
      for (uint32_t i = 0; i < (1u << 23); i++) {
        const float d = bits_f(0x3F800000u | i);
        const float q0 = d * y;
        const float q = fmaf(fmaf(-q0, s, d), y, q0);
        cases++;
        if (f_bits(q) != f_bits(d / s)) bad++;
      }
    }
    printf("pairs %lu %lu\n", bad, cases);
  }
  for (int top = 7; top <= 15; top += 8) {
    unsigned long bad = 0, cases = 0;
#pragma omp parallel for reduction(+ : bad, cases) schedule(dynamic, 64)
    for (int h = 1; h < 0x7C00; h++) {
      const float s = f16_value((uint32_t)h);
      const float y = one / s;
      for (int k = 0; k <= top; k++) {
        const float c = (float)((k + 0.5) * (double)s);    /* k = top: just past the clamp */
        const uint32_t cb = f_bits(c);
        for (int j = -1024; j <= 1024; j++) {
          const float d = bits_f(cb + (uint32_t)j);
          cases++;
          if (kernel_code(d, s, y, top) != defined_code(d, s, top)) bad++;
        }
        const float e = (float)(top * (double)s) * (float)(k + 1);   /* far above the range */
        cases++;
        if (kernel_code(e, s, y, top) != defined_code(e, s, top)) bad++;
      }
    }
    printf("ties_%d %lu %lu\n", top, bad, cases);
  }
  {
    const uint32_t hs[3] = {0x0001, 0x0400, 0x7BFF};
    unsigned long bad = 0, cases = 0;
    for (int t = 0; t < 3; t++) {
      const float s = f16_value(hs[t]), y = one / s;
      for (uint32_t i = 0; i < (1u << 23); i++) {                  /* subnormal d */
        const float d = bits_f(i);
        cases++;
        if (kernel_code(d, s, y, 15) != 0 || defined_code(d, s, 15) != 0) bad++;
      }
      const uint32_t top_bits = f_bits(s * 0.25f);
      for (uint32_t i = 0; i < (1u << 20); i++) {                  /* up to s/4 */
        const float d = bits_f(top_bits - i);
        cases++;
        if (kernel_code(d, s, y, 15) != 0 || defined_code(d, s, 15) != 0) bad++;
      }
    }
    printf("small %lu %lu\n", bad, cases);
  }
  return 0;
}
