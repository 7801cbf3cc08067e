/*
 * Exhaustive checks of the short norm and reciprocal sequences of the
 * TurboQuant encoder's common case (kvc_arch.h: sqrt_rn_normal,
 * recip_newton), evaluated with the same binary32 operations (C float,
 * -ffp-contract=off, fmaf).  The hardware square-root and reciprocal
 * estimates are accurate to one ulp, so every start s0 within one ulp of the
 * exact result is tried: the correctly rounded value and its two neighbours.
 *   1. sqrt: from s0, sd = s0 - ulp, su = s0 + ulp; take sd if
 *      fma(-sd, s0, S) <= 0, su if fma(-su, s0, S) > 0, else s0.  Every
 *      binary32 S in [2^-96, 2^31).
 *   2. reciprocal: one Newton step y0 + fma(-n, y0, 1) * y0, for every
 *      binary32 n in [2^-48, 2^16) (the norms the sums of squares above give)
 *      and every start y0 within one ulp of 1/n.  The one start per binade
 *      that the step leaves wrong -- n = (2 - 2^-23) 2^k started at 2^-(k+1),
 *      a fixed point -- is counted apart ("recip_fixed_point"); what the
 *      hardware estimate gives there is checked on the device.
 * The references are C's correctly rounded sqrtf and float division.
 * Prints one line per check: "<name> <mismatches> <cases>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t f_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

static float sqrt_corrected(float s, float S) {
  const float sd = bits_f(f_bits(s) - 1u), su = bits_f(f_bits(s) + 1u);
  const float t = fmaf(-sd, s, S) <= 0.0f ? sd : s;
  return fmaf(-su, s, S) > 0.0f ? su : t;
}

int main(void) {
  {
    const uint32_t lo = f_bits(0x1p-96f), hi = f_bits(0x1p31f);
    unsigned long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
    for (long i = lo; i < (long)hi; i++) {
      const float S = bits_f((uint32_t)i);
      const float ref = sqrtf(S);
      for (int d = -1; d <= 1; d++) {
        const float s0 = bits_f(f_bits(ref) + (uint32_t)d);
        if (f_bits(sqrt_corrected(s0, S)) != f_bits(ref)) bad++;
      }
    }
    printf("sqrt_normal %lu %ld\n", bad, 3L * (long)(hi - lo));
  }
  {
    const uint32_t lo = f_bits(0x1p-48f), hi = f_bits(0x1p16f);
    unsigned long bad = 0, fixed = 0, cases = 0;
#pragma omp parallel for reduction(+ : bad, fixed, cases) schedule(static, 1 << 16)
    for (long i = lo; i < (long)hi; i++) {
      const float n = bits_f((uint32_t)i);
      volatile float one = 1.0f;
      const float ref = one / n;
      for (int d = -1; d <= 1; d++) {
        const float y0 = bits_f(f_bits(ref) + (uint32_t)d);
        /* within one ulp of 1/n: |n y0 - 1| <= n ulp(y0), exact in double */
        int e;
        frexpf(y0, &e);
        const double u = ldexp(1.0, e - 24);
        if (fabs((double)n * (double)y0 - 1.0) > (double)n * u) continue;
        cases++;
        const float y = fmaf(fmaf(-n, y0, 1.0f), y0, y0);
        if (f_bits(y) == f_bits(ref)) continue;
        if ((f_bits(n) & 0x7FFFFFu) == 0x7FFFFFu && (f_bits(y0) & 0x7FFFFFu) == 0) fixed++;
        else bad++;
      }
    }
    printf("recip_normal %lu %lu\n", bad, cases);
    printf("recip_fixed_point %lu %ld\n", fixed, (long)((hi - lo) >> 23));
  }
  return 0;
}
