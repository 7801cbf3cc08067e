/*
 * Check of the reciprocal division in libkvc's rANS encoder
 * (kvc_ans_device.h: AnsEnc, ans_put): floor(x / f) = (x * m) >> (31 + l)
 * with l = ceil(log2 f), m = ceil(2^(31+l) / f), for every frequency f in
 * [1, 4096] -- exact for all x < 2^31 by Granlund and Montgomery (PLDI 1994,
 * Thm 4.2) -- over all x < 2^16, every x = q*f + r (r in {0, 1, f-1}) around
 * the top of the encoder's range x < 2^19 * f, and 4096 pseudo-random x per f.
 * Also that m fits 32 bits.  Prints "<mismatches> <cases>".
 */
#include <stdint.h>
#include <stdio.h>

int main(void) {
  unsigned long bad = 0, cases = 0;
  uint64_t rng = 0x9E3779B97F4A7C15ull;
  for (uint32_t f = 1; f <= 4096; f++) {
    uint32_t l = 0;
    while ((1u << l) < f) l++;
    const uint64_t m64 = ((1ull << (31 + l)) + f - 1) / f;
    if (m64 >> 32) bad++;
    const uint32_t m = (uint32_t)m64;
#define CHECK(X)                                                        \
  do {                                                                  \
    const uint32_t x_ = (X);                                            \
    cases++;                                                            \
    if ((uint32_t)(((uint64_t)x_ * m) >> (31 + l)) != x_ / f) bad++;    \
  } while (0)
    for (uint32_t x = 0; x < 65536; x++) CHECK(x);
    const uint64_t top = (uint64_t)f << 19;                    /* x < 2^19 * f <= 2^31 */
    for (uint64_t q = top / f - 2048; q < top / f; q++) {
      CHECK((uint32_t)(q * f));
      CHECK((uint32_t)(q * f + 1 < top ? q * f + 1 : q * f));
      CHECK((uint32_t)(q * f + f - 1));
    }
    for (int i = 0; i < 4096; i++) {
      rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
      CHECK((uint32_t)(rng % top));
    }
  }
  printf("%lu %lu\n", bad, cases);
  return 0;
}
