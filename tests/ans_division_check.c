/*
 * Check of the state update of libkvc's rANS encoder (kvc_ans_device.h:
 * AnsEnc, ans_put): for every frequency f in [1, 4096] and cumulative
 * frequency cum in {0, 4096 - f}, the update
 *     q = ((x * rcp) >> 32) >> shift,   x' = x + bias + q * cmpl  (mod 2^32)
 * with rcp = ceil(2^(31+l) / f), shift = l - 1, l = ceil(log2 f), bias = cum,
 * cmpl = 4096 - f for f >= 2, and rcp = 2^32 - 1, shift = 0,
 * bias = cum + 4095, cmpl = 4095 for f = 1, equals the rANS coding function
 *     C(x) = floor(x / f) * 4096 + (x mod f) + cum
 * for all x < 2^16, every x = q*f + r (r in {0, 1, f-1}) in the top 2048
 * quotients of the encoder's range x < 2^19 * f, and 4096 pseudo-random x in
 * that range per f; also that q < 2^19 (the product q * cmpl is a 24-bit
 * multiply) and that rcp fits 32 bits.  floor(x / f) = (x * rcp) >> (31 + l)
 * holds for all x < 2^31 by Granlund and Montgomery (PLDI 1994, Thm 4.2).
 * Prints "<mismatches> <cases>".
 */
#include <stdint.h>
#include <stdio.h>

int main(void) {
  unsigned long bad = 0, cases = 0;
  uint64_t rng = 0x9E3779B97F4A7C15ull;
  for (uint32_t f = 1; f <= 4096; f++) {
    uint32_t l = 0;
    while ((1u << l) < f) l++;
    uint32_t rcp, shift, cmpl = 4096 - f;
    if (f == 1) {
      rcp = 0xFFFFFFFFu;
      shift = 0;
      cmpl = 4095;
    } else {
      const uint64_t m64 = ((1ull << (31 + l)) + f - 1) / f;
      if (m64 >> 32) bad++;
      rcp = (uint32_t)m64;
      shift = l - 1;
    }
    for (int ci = 0; ci < 2; ci++) {
      const uint32_t cum = ci ? 4096 - f : 0;
      const uint32_t bias = f == 1 ? cum + 4095 : cum;
#define CHECK(X)                                                                \
  do {                                                                          \
    const uint32_t x_ = (X);                                                    \
    const uint32_t q_ = (uint32_t)(((uint64_t)x_ * rcp) >> 32) >> shift;        \
    const uint32_t y_ = x_ + bias + q_ * cmpl;                                  \
    cases++;                                                                    \
    if (y_ != (x_ / f) * 4096u + x_ % f + cum || q_ >= (1u << 19)) bad++;       \
  } while (0)
      for (uint32_t x = 1; x < 65536; x++) CHECK(x);
      const uint64_t top = (uint64_t)f << 19;                  /* x < 2^19 * f <= 2^31 */
      for (uint64_t q = top / f - 2048; q < top / f; q++) {
        CHECK((uint32_t)(q * f));
        CHECK((uint32_t)(q * f + 1 < top ? q * f + 1 : q * f));
        CHECK((uint32_t)(q * f + f - 1));
      }
      for (int i = 0; i < 4096; i++) {
        rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
        CHECK((uint32_t)(1 + rng % (top - 1)));
      }
    }
  }
  printf("%lu %lu\n", bad, cases);
  return 0;
}
