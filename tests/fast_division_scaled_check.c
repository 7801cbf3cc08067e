/*
 * Exhaustive check of the per-vector division shortcut of libkvc's encode
 * kernels (kvc_kernels.hip: div_scaled), evaluated with the same binary32
 * operations (C float with -ffp-contract=off, fmaf):
 *     RN(x / s) = q0 + e*r   with r = RN(1/s), q0 = RN(x*r), e = fma(-q0, s, x)
 * for every scale s the codecs form from a vector's absolute maximum amax
 * and every source value x with |x| <= amax (the sequence is odd in x, so
 * x >= 0 covers both signs), for BF16 and FP16 sources:
 *   int8      s = RN(max(amax, 1e-12) / 127)
 *   int8rows  s = BF16(RN(max(amax, BF16(1e-12)) / 127))
 *   fp8dyn    s = RN(max(amax, 1e-12) * RN(1/448))
 * The reference is C's correctly rounded float division.  Counted per check:
 * quotient mismatches; INT8 code mismatches, clamp(rint(q), -127, 127) of
 * the two quotients differing; and FP8 code mismatches -- quotients that
 * differ and are not both below 2^-10, the largest magnitude that E4M3FN
 * rounds to zero (half its smallest subnormal 2^-9, a tie going to the even
 * code 0; both quotients have the sign of x).
 * Prints one line per check:
 *   "<name> <quotient mismatches> <int8 code mismatches> <fp8 code mismatches> <cases>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t f_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

/* BF16 round to nearest even of a finite binary32 (the result widened) */
static float bf16_rne(float x) {
  const uint32_t b = f_bits(x);
  return bits_f(((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16) << 16);
}
/* value of a 16-bit source pattern */
static float src_value(uint32_t h, int fp16) {
  if (!fp16) return bits_f(h << 16);
  const uint32_t e = (h >> 10) & 31, m = h & 0x3FF;
  return e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
}
static float int8_code(float q) {
  float c = rintf(q);
  return c > 127.0f ? 127.0f : (c < -127.0f ? -127.0f : c);
}

enum { INT8, INT8ROWS, FP8DYN };

static void check(const char *name, int kind, int fp16) {
  const uint32_t top = fp16 ? 0x7BFF : 0x7F7F;        /* largest finite pattern */
  volatile float one = 1.0f, c127 = 127.0f, c448 = 448.0f;
  const float r448 = one / c448;
  const float floor_f32 = 1e-12f, floor_bf16 = bf16_rne(1e-12f);
  const float fp8_zero = ldexpf(1.0f, -10);
  unsigned long badq = 0, badc = 0, badf = 0, cases = 0;
#pragma omp parallel for reduction(+ : badq, badc, badf, cases) schedule(dynamic, 64)
  for (long ia = 0; ia <= (long)top; ia++) {
    const float amax = src_value((uint32_t)ia, fp16);
    float s;
    if (kind == INT8) s = fmaxf(amax, floor_f32) / c127;
    else if (kind == INT8ROWS) s = bf16_rne(fmaxf(amax, floor_bf16) / c127);
    else s = fmaxf(amax, floor_f32) * r448;
    const float r = one / s;
    for (uint32_t ix = 0; ix <= (uint32_t)ia; ix++) {
      const float x = src_value(ix, fp16);
      const float ref = x / s;
      const float q0 = x * r;
      const float q = fmaf(fmaf(-q0, s, x), r, q0);
      cases++;
      if (f_bits(q) != f_bits(ref)) {
        badq++;
        if (int8_code(q) != int8_code(ref)) badc++;
        if (!(q < fp8_zero && ref < fp8_zero)) badf++;
      }
    }
  }
  printf("%s %lu %lu %lu %lu\n", name, badq, badc, badf, cases);
  fflush(stdout);
}

int main(void) {
  check("int8_bf16", INT8, 0);
  check("int8_fp16", INT8, 1);
  check("int8rows_bf16", INT8ROWS, 0);
  check("int8rows_fp16", INT8ROWS, 1);
  check("fp8dyn_bf16", FP8DYN, 0);
  check("fp8dyn_fp16", FP8DYN, 1);
  return 0;
}
