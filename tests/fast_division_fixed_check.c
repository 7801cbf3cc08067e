/*
 * Check of the FP8 fixed-scale division shortcut of libkvc's encode kernels
 * (kvc_kernels.hip: div_scaled with the caller's scale), evaluated with the
 * same binary32 operations (C float with -ffp-contract=off, fmaf):
 *     RN(x / s) = q0 + e*r   with r = RN(1/s), q0 = RN(x*r), e = fma(-q0, s, x)
 * The kernels take this path for fixed scales s in [2^-60, 2^60] (the IEEE
 * division otherwise).  There q0 is a faithful quotient, the remainder e is
 * exact (no underflow: a quotient of 2^-10 or more needs |x| >= 2^-70) and
 * r is the correctly rounded reciprocal, so by Markstein's theorem (one FMA
 * correction of a faithful quotient with a correctly rounded reciprocal gives
 * the correctly rounded quotient) the result is RN(x / s).  This program
 * checks it on every source value 0 <= x <= 448 (larger ones send an FP8
 * segment raw; the sequence is odd in x) of BF16 and of FP16 against 256
 * scales per binade of [2^-60, 2^60): the significands 0, 1, 2, 3, 2^22,
 * 2^23 - 1, 2^23 - 2, the repeating 0101.. and 1010.. patterns and 247
 * pseudo-random ones (xorshift32), plus s = 2^60.
 * Counted: quotients that differ from C's correctly rounded division and are
 * not both at most 2^-10 (E4M3FN rounds those to zero: half its smallest
 * subnormal, a tie going to the even code 0).
 * Prints "<name> <mismatches> <cases>" for bf16 and fp16.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t f_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

static float src_value(uint32_t h, int fp16) {
  if (!fp16) return bits_f(h << 16);
  const uint32_t e = (h >> 10) & 31, m = h & 0x3FF;
  return e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
}

enum { kPerBinade = 256, kLo = -60, kHi = 60 };

static uint32_t scale_bits(int binade, int i) {
  static const uint32_t fixed_sig[9] = {0, 1, 2, 3, 0x400000, 0x7FFFFF, 0x7FFFFE, 0x555555, 0x2AAAAA};
  uint32_t sig;
  if (i < 9) {
    sig = fixed_sig[i];
  } else {
    uint32_t st = 0x9E3779B9u ^ (uint32_t)(binade * 7919 + i * 104729);
    for (int k = 0; k < 4; k++) {
      st ^= st << 13;
      st ^= st >> 17;
      st ^= st << 5;
    }
    sig = st & 0x7FFFFF;
  }
  return ((uint32_t)(binade + 127) << 23) | sig;
}

static void check(const char *name, int fp16) {
  const uint32_t top = fp16 ? 0x5F00 : 0x43E0;        /* 448 */
  const float fp8_zero = ldexpf(1.0f, -10);
  volatile float one = 1.0f;
  const long nscales = (long)(kHi - kLo) * kPerBinade + 1;
  unsigned long bad = 0, cases = 0;
#pragma omp parallel for reduction(+ : bad, cases) schedule(dynamic, 16)
  for (long is = 0; is < nscales; is++) {
    const float s = is + 1 == nscales ? ldexpf(1.0f, kHi)
                                      : bits_f(scale_bits(kLo + (int)(is / kPerBinade), (int)(is % kPerBinade)));
    const float r = one / s;
    for (uint32_t ix = 0; ix <= top; ix++) {
      const float x = src_value(ix, fp16);
      const float ref = x / s;
      const float q0 = x * r;
      const float q = fmaf(fmaf(-q0, s, x), r, q0);
      cases++;
      if (f_bits(q) != f_bits(ref) && !(q <= fp8_zero && ref <= fp8_zero)) bad++;
    }
  }
  printf("%s %lu %lu\n", name, bad, cases);
  fflush(stdout);
}

int main(void) {
  check("fixed_bf16", 0);
  check("fixed_fp16", 1);
  return 0;
}
