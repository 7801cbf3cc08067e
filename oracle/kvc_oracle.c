/*
 * kvc_oracle.c -- plain scalar CPU oracle for the paged KV-cache codecs.
 *
 * TEST INFRASTRUCTURE ONLY (see kvc_oracle.h).  Build:
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC \
 *       -o libkvc_oracle.so kvc_oracle.c -lm
 * x86-64 evaluates float expressions in binary32 (SSE, FLT_EVAL_METHOD 0),
 * so each C float operation below is exactly one RN binary32 operation.
 *
 * Citations name the page and its section:
 *   [OKV-SF] OrbitKV "KV precision and storage encoding":
 *            "FP8 and TurboQuant" (E4M3FN RNE with signed zero and
 *            subnormals; nonfinite or |x|>448 segments stay raw; TurboQuant K
 *            = normalize, deterministic random signs, orthonormal WHT,
 *            Gaussian Lloyd-Max centroids, norm-corrected inverse with the
 *            original FP16 norm; V = b-bit codes per vector against an FP16
 *            minimum and scale; D in {32,64,128,256}; 66/68 and 50/52 byte
 *            payloads at D=128) and "Ownership, storage and GDS" (segment
 *            carries version, original length, format, stored length, CRC32;
 *            keep only when the aligned footprint saves >= 12.5%; sources up
 *            to 16 MiB are encoded) and "GPU ANS" (lossless entropy coding
 *            of typed 16-bit pages; decompression checks the exact output
 *            length; incompressible pages stay raw; at least 4 KiB of
 *            input).
 *   [HIQ]    "Building a quantized HiCache for SGLang": "Building the INT8
 *            codec" (symmetric per-head INT8: amax floor, scale = amax/127,
 *            FP32 quotient, round, clamp to +-127; all-zero head restores
 *            to exact zero) and "Why exactly 1,152 bytes?" (a token's K or
 *            V row: H x D INT8 codes, then H BF16 scales, padded to a
 *            multiple of 128 bytes).
 *   [KNLP]   "Asymmetric KV: methods and results": "Precision and scaling
 *            reference" (FP32 amax clamped at 1e-12, times the rounded FP32
 *            reciprocal of 448, FP32 divide, clip to +-448, E4M3FN RNE;
 *            dynamic = per token/head vector; FP32 scales).
 */
#define _GNU_SOURCE
#include "kvc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define SLOT_ALIGN 256u
#define HEADER_BYTES 32u
#define MAX_SEGMENT_BYTES (16u << 20)
#define MAX_D 256
#define ROWS_OFFSET 128u    /* INT8_ROWS: the rows start 128 bytes into the slot */
/* ANS16: 64 interleaved rANS streams per byte plane, 12-bit probabilities,
 * 32-bit state in [2^23, 2^31), byte-wise renormalisation */
#define ANS_STREAMS 64u
#define ANS_PROB_BITS 12
#define ANS_M (1u << ANS_PROB_BITS)
#define ANS_L (1u << 23)
#define ANS_MIN_BYTES 4096u
#define ANS_MAX_BYTES 32768u
#define FLAG_HEAP 16        /* stored bytes sit at spill_offset, outside the slot */

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* BF16 is the upper half of a binary32 pattern: widening is exact. */
float kvo_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float kvo_f16_to_f32(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) {
    if (m) return s ? -NAN : NAN;
    return s ? -INFINITY : INFINITY;
  }
  if (e == 0) v = ldexp((double)m, -24);              /* subnormal */
  else        v = ldexp((double)(1024 + m), e - 25);  /* normal    */
  return (float)(s ? -v : v);                         /* exact     */
}

/* Nearest value of a binary format with p significand bits (hidden bit
 * included) and minimum normal exponent emin, ties to the even significand.
 * x / quantum and rint(.) * quantum are exact in double; rint rounds to
 * nearest-even in the default rounding mode.  No overflow handling here. */
static double round_to_format(double x, int p, int emin) {
  int e;
  if (x == 0.0) return x;
  frexp(fabs(x), &e);          /* |x| = f * 2^e, f in [0.5, 1) */
  int ex = e - 1;              /* floor(log2 |x|)               */
  if (ex < emin) ex = emin;    /* subnormal range: fixed quantum */
  double quantum = ldexp(1.0, ex - (p - 1));
  return rint(x / quantum) * quantum;
}

uint16_t kvo_f32_to_bf16(float x) {
  if (isnan(x)) return signbit(x) ? 0xFFC0 : 0x7FC0;
  double q = round_to_format((double)x, 8, -126);
  if (fabs(q) >= ldexp(1.0, 128)) q = signbit(x) ? -INFINITY : INFINITY;
  float f = (float)q;          /* exact: q is a bf16 value or infinity */
  if (f == 0.0f && signbit(x)) f = -0.0f;
  return (uint16_t)(f2u(f) >> 16);
}

uint16_t kvo_f32_to_f16(float x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return s | 0x7E00;
  double q = round_to_format((double)x, 11, -14);
  double a = fabs(q);
  if (a >= 65536.0) return s | 0x7C00;          /* rounds past 65504 */
  if (a == 0.0) return s;
  int e;
  frexp(a, &e);
  int ex = e - 1;
  if (ex < -14) return s | (uint16_t)(a / ldexp(1.0, -24));   /* subnormal */
  int mant = (int)(a / ldexp(1.0, ex - 10)) - 1024;
  return s | (uint16_t)((ex + 15) << 10) | (uint16_t)mant;
}

/* OCP OFP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 448; subnormals step 2^-9.
 * Precondition |x| <= 448 (the codecs gate or clip before converting). */
uint8_t kvo_f32_to_e4m3(float x) {
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  if (isnan(x) || fabs((double)x) > 448.0) return s | 0x7F;
  double q = round_to_format((double)x, 4, -6);
  double a = fabs(q);
  if (a == 0.0) return s;                       /* signed zero kept */
  int e;
  frexp(a, &e);
  int ex = e - 1;
  if (ex < -6) return s | (uint8_t)(a / ldexp(1.0, -9));      /* subnormal */
  int mant = (int)(a / ldexp(1.0, ex - 3)) - 8;
  return s | (uint8_t)((ex + 7) << 3) | (uint8_t)mant;
}

float kvo_e4m3_to_f32(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return s ? -NAN : NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)(s ? -v : v);
}

/* Brute force: the nearest of the finite E4M3FN codes of the same sign as x;
 * among equidistant candidates the one with an even code (mantissa LSB 0). */
uint8_t kvo_e4m3_nearest_search(float x) {
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  double ax = fabs((double)x);
  int best = -1;
  double bestd = 0.0;
  for (int c = 0; c < 0x7F; c++) {
    double d = fabs((double)kvo_e4m3_to_f32((uint8_t)c) - ax);
    if (best < 0 || d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return s | (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* Method constants                                                         */
/* ------------------------------------------------------------------------ */

static double std_pdf(double t) { return exp(-0.5 * t * t) / sqrt(2.0 * 3.14159265358979323846); }
static double std_upper_tail(double t) { return 0.5 * erfc(t / sqrt(2.0)); }

/* Lloyd-Max scalar quantizer for the standard Gaussian [OKV-SF "FP8 and
 * TurboQuant": "Gaussian Lloyd-Max centroids"].  The optimal quantizer is a
 * fixed point of (1) thresholds at midpoints of neighbouring centroids and
 * (2) each centroid the conditional mean of its cell:
 *     c = (pdf(lo) - pdf(hi)) / (P(X > lo) - P(X > hi)).
 * The quantizer is symmetric, so only the positive half is iterated; the
 * middle threshold is exactly 0. */
int kvo_lloyd_max(int bits, double *centroids, double *thresholds) {
  int n = 1 << bits, m = n / 2, it;
  double pc[128], tb[129];
  for (int j = 0; j < m; j++) pc[j] = (j + 0.5) * 3.0 / m;
  for (it = 1; it <= 2000000; it++) {
    double maxd = 0.0;
    tb[0] = 0.0;
    for (int j = 1; j < m; j++) tb[j] = 0.5 * (pc[j - 1] + pc[j]);
    for (int j = 0; j < m; j++) {
      double lo = tb[j];
      double num, den;
      if (j == m - 1) {
        num = std_pdf(lo);
        den = std_upper_tail(lo);
      } else {
        double hi = tb[j + 1];
        num = std_pdf(lo) - std_pdf(hi);
        den = std_upper_tail(lo) - std_upper_tail(hi);
      }
      double c = num / den;
      double dd = fabs(c - pc[j]);
      if (dd > maxd) maxd = dd;
      pc[j] = c;
    }
    if (maxd < 1e-15) break;
  }
  for (int j = 0; j < m; j++) {
    centroids[m + j] = pc[j];
    centroids[m - 1 - j] = -pc[j];
  }
  for (int k = 0; k < n - 1; k++) thresholds[k] = 0.5 * (centroids[k] + centroids[k + 1]);
  thresholds[m - 1] = 0.0;
  return it;
}

/* The FP32 tables for 1..4 bits are computed once when the library loads
 * (the fixed-point iteration takes milliseconds). */
static float g_cent[5][16], g_thr[5][15];

__attribute__((constructor)) static void kvo_init_codebooks(void) {
  double c[16], t[15];
  for (int bits = 1; bits <= 4; bits++) {
    int n = 1 << bits;
    kvo_lloyd_max(bits, c, t);
    for (int k = 0; k < n; k++) g_cent[bits][k] = (float)c[k];
    for (int k = 0; k < n - 1; k++) g_thr[bits][k] = (float)t[k];
  }
}

void kvo_codebook_f32(int bits, float *centroids, float *thresholds) {
  int n = 1 << bits;
  for (int k = 0; k < n; k++) centroids[k] = g_cent[bits][k];
  for (int k = 0; k < n - 1; k++) thresholds[k] = g_thr[bits][k];
}

/* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): state += golden gamma, then the variant-13
 * finaliser. */
uint64_t kvo_splitmix64_next(uint64_t *state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* "deterministic random signs" [OKV-SF "FP8 and TurboQuant"]; the generator
 * is versioned and our own ("OrbitKV's versioned sign generator ... are its
 * own").  Version 1: one sign vector per (seed, D), shared by every layer,
 * head and token. */
void kvo_signs(uint64_t seed, int d, int8_t *sigma) {
  uint64_t st = seed;
  for (int i = 0; i < d; i++) sigma[i] = (kvo_splitmix64_next(&st) >> 63) ? -1 : 1;
}

/* ------------------------------------------------------------------------ */
/* Vector building blocks                                                   */
/* ------------------------------------------------------------------------ */

/* Unnormalised Walsh-Hadamard transform in Sylvester (natural) order: the
 * matrix H_{2n} = [[H_n, H_n], [H_n, -H_n]]; stage h pairs i and i+h. */
void kvo_wht_f32(float *v, int d) {
  for (int h = 1; h < d; h *= 2)
    for (int i = 0; i < d; i++)
      if (!(i & h)) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

/* sum of squares as a pairwise tree: leaves RN(x_i^2), then adjacent pairs,
 * then adjacent pairs of pairs, ... */
float kvo_sumsq_tree(const float *x, int d) {
  float s[MAX_D];
  for (int i = 0; i < d; i++) s[i] = x[i] * x[i];
  for (int w = d; w > 1; w /= 2)
    for (int i = 0; i < w / 2; i++) s[i] = s[2 * i] + s[2 * i + 1];
  return s[0];
}

static float src_to_f32(uint16_t h, int dtype) {
  return dtype == KVO_BF16 ? kvo_bf16_to_f32(h) : kvo_f16_to_f32(h);
}
static uint16_t f32_to_out(float x, int dtype) {
  return dtype == KVO_BF16 ? kvo_f32_to_bf16(x) : kvo_f32_to_f16(x);
}

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) { uint32_t v = 0; for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i); return v; }
static uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i); return v; }

static int codec_bits(int codec) {
  switch (codec) {
    case KVO_UNIFORM3: case KVO_TQ3: return 3;
    case KVO_UNIFORM4: case KVO_TQ4: return 4;
    case KVO_RAW: return 16;
    default: return 8;
  }
}

/* code k of a vector: LSB-first bit stream, element i at bits [b*i, b*i+b) */
static void put_code(uint8_t *blk, int i, int b, unsigned code) {
  for (int k = 0; k < b; k++) {
    int bit = b * i + k;
    if ((code >> k) & 1u) blk[bit >> 3] |= (uint8_t)(1u << (bit & 7));
  }
}
static unsigned get_code(const uint8_t *blk, int i, int b) {
  unsigned c = 0;
  for (int k = 0; k < b; k++) {
    int bit = b * i + k;
    c |= (unsigned)((blk[bit >> 3] >> (bit & 7)) & 1u) << k;
  }
  return c;
}

/* ------------------------------------------------------------------------ */
/* Format sizes                                                             */
/* ------------------------------------------------------------------------ */

int kvo_code_bytes(int codec, int d) { return codec_bits(codec) * d / 8; }

int kvo_meta_bytes(int codec) {
  switch (codec) {
    case KVO_FP8_DYNAMIC: case KVO_INT8: return 4;          /* FP32 scale   */
    case KVO_UNIFORM3: case KVO_UNIFORM4: return 4;         /* FP16 min, scale */
    case KVO_TQ3: case KVO_TQ4: return 2;                   /* FP16 norm    */
    default: return 0;                                      /* raw, FP8 direct/fixed */
  }
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

/* [HIQ "Why exactly 1,152 bytes?"]: one token's row of the INT8 record
 * codec -- heads*d INT8 codes and heads BF16 scales (1,040 bytes at 8 x 128),
 * padded to the next multiple of 128 bytes (1,152 = 9 x 128). */
size_t kvo_row_bytes(int d, int heads) {
  return align_up((size_t)heads * (size_t)d + 2u * (size_t)heads, 128);
}

size_t kvo_slot_bytes(int codec, int d, int n_vec, int heads) {
  if (codec == KVO_ANS16) return align_up(HEADER_BYTES, SLOT_ALIGN);   /* the payload goes to the spill region */
  if (codec == KVO_INT8_ROWS)
    return align_up(ROWS_OFFSET + (size_t)(n_vec / heads) * kvo_row_bytes(d, heads), SLOT_ALIGN);
  size_t payload = (size_t)n_vec * (size_t)(kvo_code_bytes(codec, d) + kvo_meta_bytes(codec));
  return align_up(HEADER_BYTES + payload, SLOT_ALIGN);
}

/* [OKV-SF "Ownership, storage and GDS"]: keep an encoded segment only when
 * its aligned footprint saves at least 12.5%; segments above 16 MiB stay raw.
 * [OKV-SF "FP8 and TurboQuant"]: protected layers stay exact. */
int kvo_effective_codec(int codec, int d, int n_vec, int heads, int is_protected) {
  size_t orig = (size_t)n_vec * (size_t)d * 2;
  if (is_protected || codec == KVO_RAW) return KVO_RAW;
  if (orig > MAX_SEGMENT_BYTES) return KVO_RAW;
  /* [OKV-SF "GPU ANS"]: at least 4 KiB of input; the kernels hold at most
   * 32 KiB of a segment */
  if (codec == KVO_ANS16 && (orig < ANS_MIN_BYTES || orig > ANS_MAX_BYTES)) return KVO_RAW;
  if (8 * kvo_slot_bytes(codec, d, n_vec, heads) > 7 * orig) return KVO_RAW;
  return codec;
}

/* ------------------------------------------------------------------------ */
/* Per-vector encoders.  Return 1 if the vector forces the segment raw.      */
/* ------------------------------------------------------------------------ */

/* [OKV-SF "FP8 and TurboQuant"] direct cast, no scale. */
static int enc_fp8_direct(const float *x, int d, uint8_t *codes) {
  for (int i = 0; i < d; i++) codes[i] = kvo_f32_to_e4m3(x[i]);
  return 0;
}

/* [KNLP "Precision and scaling reference"]: q = RN(x / s), clip to +-448,
 * E4M3FN RNE. */
static void enc_fp8_scaled(const float *x, int d, float s, uint8_t *codes) {
  for (int i = 0; i < d; i++) {
    float q = x[i] / s;
    if (q > 448.0f) q = 448.0f;
    if (q < -448.0f) q = -448.0f;
    codes[i] = kvo_f32_to_e4m3(q);
  }
}

/* [KNLP]: dynamic scale per token/head vector:
 * s = RN(max(amax, 1e-12) * RN(1/448)). */
static float fp8_dynamic_scale(const float *x, int d) {
  float amax = 0.0f;
  for (int i = 0; i < d; i++) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  if (amax < 1e-12f) amax = 1e-12f;
  const float r448 = 1.0f / 448.0f;
  return amax * r448;
}

/* [HIQ "Building the INT8 codec"]: amax clamped below at the floor (1e-12),
 * scale = RN(amax / 127) kept in FP32, q = RNE(RN(x / scale)), clamp +-127. */
static float int8_scale(const float *x, int d) {
  float amax = 0.0f;
  for (int i = 0; i < d; i++) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  if (amax < 1e-12f) amax = 1e-12f;
  return amax / 127.0f;
}
/* [HIQ "Building the INT8 codec"], record form: the same steps on BF16
 * tensors -- amax (a BF16 value) clamped below at the floor, the floor
 * itself a BF16 value (1e-12 rounded to BF16); scale = amax / 127 computed
 * in FP32 and rounded to BF16; quotient formed in FP32 against that BF16
 * scale, rounded half to even, clamped to +-127. */
static float int8_rows_scale(const float *x, int d) {
  const float floor_bf16 = kvo_bf16_to_f32(kvo_f32_to_bf16(1e-12f));
  float amax = 0.0f;
  for (int i = 0; i < d; i++) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  if (amax < floor_bf16) amax = floor_bf16;
  return kvo_bf16_to_f32(kvo_f32_to_bf16(amax / 127.0f));
}
static void enc_int8(const float *x, int d, float s, uint8_t *codes) {
  for (int i = 0; i < d; i++) {
    float q = rintf(x[i] / s);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    codes[i] = (uint8_t)(int8_t)q;
  }
}

/* [OKV-SF "FP8 and TurboQuant"] V: per-vector uniform b-bit quantization with
 * an FP16 minimum and an FP16 scale.  sigma = RN(RN(max - min) / (2^b - 1));
 * both are stored as FP16, and the codes are taken against the stored values
 * so that encoder and decoder agree:
 *   code = clamp(RNE(RN(RN(x - m_h) / sigma_h)), 0, 2^b - 1),
 * the binary32 quotient rounded once to binary32 and then to the nearest
 * integer, ties to even.  sigma_h == 0 gives all-zero codes. */
static int enc_uniform(const float *x, int d, int bits, uint8_t *codes, uint8_t *meta) {
  int top = (1 << bits) - 1;
  float mn = x[0], mx = x[0];
  for (int i = 1; i < d; i++) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  /* min and max are values, and a zero extreme is +0 whatever the signs of
   * the zeros in the vector (x + 0 turns -0 into +0, nothing else) */
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  float sig = (mx - mn) / (float)top;
  uint16_t mh = kvo_f32_to_f16(mn), sh = kvo_f32_to_f16(sig);
  float mhf = kvo_f16_to_f32(mh), shf = kvo_f16_to_f32(sh);
  put_u16(meta, mh);
  put_u16(meta + 2, sh);
  if (!isfinite(mhf) || !isfinite(shf)) return 1;
  memset(codes, 0, (size_t)(bits * d / 8));
  if (shf == 0.0f) return 0;
  for (int i = 0; i < d; i++) {
    float dd = x[i] - mhf;
    float q = dd / shf;
    float c = rintf(q);
    if (c < 0.0f) c = 0.0f;
    if (c > (float)top) c = (float)top;
    put_code(codes, i, bits, (unsigned)c);
  }
  return 0;
}

/* [OKV-SF "FP8 and TurboQuant"] K: normalise, deterministic random signs,
 * orthonormal WHT, Gaussian Lloyd-Max codes.
 *   1. ss = pairwise tree of RN(x_i^2); n = RN(sqrt(ss)); n_h = FP16(n).
 *   2. u_i = RN(x_i * RN(1/n))  (u = 0 when n == 0).
 *   3. v_i = sigma_i * u_i.
 *   4. z = unnormalised WHT(v).  The orthonormal transform is WHT/sqrt(D);
 *      a rotated unit vector has coordinates of variance 1/D, so z (which is
 *      sqrt(D) times the orthonormal output) is compared with the N(0,1)
 *      codebook directly.
 *   5. code_i = #{k : B_k < z_i}  (a value equal to a threshold takes the
 *      lower cell). */
static int enc_tq(const float *x, int d, int bits, const int8_t *sigma,
                  const float *thr, uint8_t *codes, uint8_t *meta) {
  int nthr = (1 << bits) - 1;
  float v[MAX_D];
  float ss = kvo_sumsq_tree(x, d);
  float n = sqrtf(ss);
  uint16_t nh = kvo_f32_to_f16(n);
  put_u16(meta, nh);
  if (!isfinite(kvo_f16_to_f32(nh))) return 1;
  if (n == 0.0f) {
    for (int i = 0; i < d; i++) v[i] = 0.0f;
  } else {
    float r = 1.0f / n;
    for (int i = 0; i < d; i++) {
      float u = x[i] * r;
      v[i] = sigma[i] < 0 ? -u : u;
    }
  }
  kvo_wht_f32(v, d);
  memset(codes, 0, (size_t)(bits * d / 8));
  for (int i = 0; i < d; i++) {
    unsigned c = 0;
    for (int k = 0; k < nthr; k++) if (thr[k] < v[i]) c++;
    put_code(codes, i, bits, c);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-vector decoders                                                      */
/* ------------------------------------------------------------------------ */

/* TurboQuant K restore [OKV-SF "FP8 and TurboQuant"]: centroid vector c_hat,
 * its norm q = tree sum of RN(c_hat_i^2), w = WHT(c_hat) (the inverse of the
 * orthonormal transform up to the factor sqrt(D)), norm correction
 * g = RN(n_h / RN(RN(sqrt(q)) * RN(sqrt(D)))), x_hat_i = sigma_i * RN(w_i * g),
 * rounded to the output type. */
static void dec_tq(const uint8_t *codes, const uint8_t *meta, int d, int bits,
                   const int8_t *sigma, const float *cent, int dtype, uint16_t *out) {
  float c[MAX_D], w[MAX_D];
  for (int i = 0; i < d; i++) c[i] = cent[get_code(codes, i, bits)];
  float q = kvo_sumsq_tree(c, d);
  memcpy(w, c, sizeof(float) * (size_t)d);
  kvo_wht_f32(w, d);
  float rd = sqrtf((float)d);
  float den = sqrtf(q) * rd;
  float g = kvo_f16_to_f32(get_u16(meta)) / den;
  for (int i = 0; i < d; i++) {
    float y = w[i] * g;
    if (sigma[i] < 0) y = -y;
    out[i] = f32_to_out(y, dtype);
  }
}

static void dec_uniform(const uint8_t *codes, const uint8_t *meta, int d, int bits,
                        int dtype, uint16_t *out) {
  float mhf = kvo_f16_to_f32(get_u16(meta));
  float shf = kvo_f16_to_f32(get_u16(meta + 2));
  for (int i = 0; i < d; i++) {
    float t = (float)get_code(codes, i, bits) * shf;   /* exact */
    out[i] = f32_to_out(mhf + t, dtype);
  }
}

/* ------------------------------------------------------------------------ */
/* Lossless entropy coding: rANS over byte planes (KVO_ANS16)               */
/* ------------------------------------------------------------------------ */

/* [OKV-SF "GPU ANS"] typed 16-bit pages are entropy coded losslessly.  The
 * coder here is range asymmetric numeral systems (rANS, J. Duda, "Asymmetric
 * numeral systems", arXiv:1311.2540, 2013) with a static model per plane:
 *   - plane 0 holds the low byte of each 16-bit value, plane 1 the high
 *     byte, in canonical element order;
 *   - element i belongs to stream (i / 8) mod 64; a stream codes its
 *     elements in increasing i;
 *   - a plane serialises as a 16-byte header (u16 mode, u16 K, 12 zero
 *     bytes), then
 *       mode 0 (raw):  the n bytes;
 *       mode 1 (rANS): a 32-byte bitmap of the K symbols present, their u16
 *                      frequencies in increasing symbol order, 64 u16 stream
 *                      lengths, the streams in stream order, each as [final
 *                      state, u32 little-endian][renormalisation bytes, last
 *                      emitted first];
 *     zero-padded to a multiple of 16 bytes, so that a plane -- and a raw
 *     plane's bytes -- start 16-byte aligned.  rANS is used when it is
 *     shorter than the raw plane. */

/* Frequencies summing to 2^12 from counts over n symbols: each present
 * symbol gets 1 plus its share of the remaining 4096 - K (K present
 * symbols), floored; the rounding remainder goes to the most frequent
 * symbol (the lowest on ties). */
void kvo_ans_normalize(const uint32_t *count, uint32_t n, uint16_t *freq) {
  uint32_t k = 0, best = 0;
  for (int s = 0; s < 256; s++) {
    if (count[s]) k++;
    if (count[s] > count[best]) best = (uint32_t)s;
  }
  uint32_t sum = 0;
  for (int s = 0; s < 256; s++) {
    freq[s] = count[s] ? (uint16_t)(1 + (uint32_t)(((uint64_t)count[s] * (ANS_M - k)) / n)) : 0;
    sum += freq[s];
  }
  if (n) freq[best] = (uint16_t)(freq[best] + (ANS_M - sum));
}

/* the rANS body of a plane (from the bitmap on); returns its size */
static size_t ans_rans_body(const uint8_t *sym, size_t n, uint8_t *out, uint32_t *k_out) {
  uint32_t count[256] = {0};
  uint16_t freq[256];
  uint32_t cum[257];
  for (size_t i = 0; i < n; i++) count[sym[i]]++;
  kvo_ans_normalize(count, (uint32_t)n, freq);
  cum[0] = 0;
  for (int s = 0; s < 256; s++) cum[s + 1] = cum[s] + freq[s];
  memset(out, 0, 32);
  uint8_t *q = out + 32;
  uint32_t k = 0;
  for (int s = 0; s < 256; s++)
    if (freq[s]) {
      out[s >> 3] |= (uint8_t)(1u << (s & 7));
      put_u16(q, freq[s]);
      q += 2;
      k++;
    }
  *k_out = k;
  uint8_t *lens = q, *dst = q + 2 * ANS_STREAMS;
  static __thread uint8_t emitted[2 * 16384];  /* per stream: at most 2 bytes per symbol */
  static __thread size_t idx[16384];
  for (uint32_t j = 0; j < ANS_STREAMS; j++) {
    /* the stream's elements: chunks c = j, j + 64, ... of 8 elements */
    size_t m = 0;
    for (size_t c = j; 8 * c < n; c += ANS_STREAMS)
      for (size_t e = 0; e < 8 && 8 * c + e < n; e++) idx[m++] = 8 * c + e;
    uint32_t x = ANS_L;
    size_t ne = 0;
    for (size_t t = m; t-- > 0;) {           /* rANS encodes in reverse */
      const uint32_t s = sym[idx[t]], f = freq[s];
      const uint32_t x_max = ((ANS_L >> ANS_PROB_BITS) << 8) * f;
      while (x >= x_max) {
        emitted[ne++] = (uint8_t)(x & 0xFF);
        x >>= 8;
      }
      x = (x / f) * ANS_M + (x % f) + cum[s];
    }
    put_u32(dst, x);
    for (size_t b = 0; b < ne; b++) dst[4 + b] = emitted[ne - 1 - b];
    put_u16(lens + 2 * j, (uint16_t)(4 + ne));
    dst += 4 + ne;
  }
  return (size_t)(dst - out);
}

/* Size of the rANS body (bitmap, frequencies, stream lengths, streams) of n
 * symbols, n <= 16384, whether or not it is shorter than n. */
size_t kvo_ans_coded_body(const uint8_t *sym, size_t n) {
  if (n > 16384) return 0;
  uint8_t *buf = (uint8_t *)malloc(1024 + 2 * n);
  if (!buf) return 0;
  uint32_t k = 0;
  const size_t body = ans_rans_body(sym, n, buf, &k);
  free(buf);
  return body;
}

/* Encode n symbols (n <= 2^20); returns the serialised size, a multiple of
 * 16 (out must hold 16 + 32 + 512 + 128 + 4 * 64 + 2 * n + 15 bytes: a
 * symbol emits at most two bytes). */
size_t kvo_ans_encode_plane(const uint8_t *sym, size_t n, uint8_t *out) {
  if (n > ((size_t)1 << 20)) return 0;
  uint32_t k = 0;
  memset(out, 0, 16);
  size_t body = ans_rans_body(sym, n, out + 16, &k);
  size_t size;
  if (body < n) {
    put_u16(out, 1);
    put_u16(out + 2, (uint16_t)k);
    size = 16 + body;
  } else {
    memcpy(out + 16, sym, n);
    size = 16 + n;
  }
  while (size & 15) out[size++] = 0;
  return size;
}

/* Decode n symbols from `in` (avail bytes).  Returns the bytes consumed, or
 * 0 on any inconsistency: an unknown mode, a bitmap not holding K symbols,
 * frequencies not summing to 2^12, a stream whose starting state lies outside
 * the coder's state interval [2^23, 2^31) (every final state of the encoder
 * lies in it), a stream running past its length or not ending exactly at its
 * length in the initial state (the exact-length check), nonzero padding. */
size_t kvo_ans_decode_plane(const uint8_t *in, size_t avail, size_t n, uint8_t *sym) {
  if (avail < 16) return 0;
  const uint32_t mode = get_u16(in), k = get_u16(in + 2);
  for (int b = 4; b < 16; b++)
    if (in[b]) return 0;
  size_t off;
  if (mode == 0) {
    if (k || avail < 16 + n) return 0;
    memcpy(sym, in + 16, n);
    off = 16 + n;
  } else if (mode == 1) {
    if (avail < 16 + 32 + 2 * (size_t)k + 2 * ANS_STREAMS) return 0;
    uint16_t freq[256];
    uint32_t cum[257], sum = 0, present = 0;
    const uint8_t *fq = in + 48;
    for (int s = 0; s < 256; s++) {
      freq[s] = 0;
      if ((in[16 + (s >> 3)] >> (s & 7)) & 1) {
        if (present == k) return 0;
        freq[s] = get_u16(fq + 2 * present++);
        if (!freq[s]) return 0;
      }
    }
    if (present != k) return 0;
    cum[0] = 0;
    for (int s = 0; s < 256; s++) {
      cum[s + 1] = cum[s] + freq[s];
      sum += freq[s];
    }
    if (sum != ANS_M) return 0;
    const uint8_t *lens = fq + 2 * k;
    off = (size_t)(lens - in) + 2 * ANS_STREAMS;
    for (uint32_t j = 0; j < ANS_STREAMS; j++) {
      const size_t len = get_u16(lens + 2 * j);
      if (len < 4 || off + len > avail) return 0;
      const uint8_t *st = in + off;
      uint32_t x = get_u32(st);
      if (x < ANS_L || x >= (ANS_L << 8)) return 0;
      size_t pos = 4;
      for (size_t c = j; 8 * c < n; c += ANS_STREAMS)
        for (size_t e = 0; e < 8 && 8 * c + e < n; e++) {
          const uint32_t slot = x & (ANS_M - 1);
          int s = 0;
          while (cum[s + 1] <= slot) s++;        /* the symbol whose interval holds the slot */
          sym[8 * c + e] = (uint8_t)s;
          x = freq[s] * (x >> ANS_PROB_BITS) + slot - cum[s];
          while (x < ANS_L) {
            if (pos >= len) return 0;
            x = (x << 8) | st[pos++];
          }
        }
      if (pos != len || x != ANS_L) return 0;
      off += len;
    }
  } else {
    return 0;
  }
  while (off & 15) {
    if (off >= avail || in[off]) return 0;
    off++;
  }
  return off;
}

/* both planes of n 16-bit values; returns the payload size */
static size_t ans_encode_segment(const uint16_t *vec, size_t n, uint8_t *out) {
  uint8_t *plane = (uint8_t *)malloc(n);
  size_t total = 0;
  for (int p = 0; p < 2; p++) {
    for (size_t i = 0; i < n; i++) plane[i] = (uint8_t)(vec[i] >> (8 * p));
    total += kvo_ans_encode_plane(plane, n, out + total);
  }
  free(plane);
  return total;
}
static int ans_decode_segment(const uint8_t *in, size_t stored, size_t n, uint16_t *out) {
  uint8_t *plane = (uint8_t *)malloc(n);
  size_t used = 0;
  int ok = 1;
  for (size_t i = 0; i < n; i++) out[i] = 0;
  for (int p = 0; p < 2 && ok; p++) {
    const size_t u = kvo_ans_decode_plane(in + used, stored - used, n, plane);
    if (!u) ok = 0;
    used += u;
    for (size_t i = 0; i < n && ok; i++) out[i] = (uint16_t)(out[i] | (plane[i] << (8 * p)));
  }
  free(plane);
  return ok && used == stored;                 /* exact length */
}

/* ------------------------------------------------------------------------ */
/* Segments                                                                 */
/* ------------------------------------------------------------------------ */

/* [OKV-SF "Ownership, storage and GDS"] a segment carries a CRC32.  The
 * common CRC-32 (reflected polynomial 0xEDB88320, register preset to all
 * ones, result complemented), bit by bit. */
uint32_t kvo_crc32(const uint8_t *p, size_t n) {
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; i++) {
    c ^= p[i];
    for (int k = 0; k < 8; k++) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
  }
  return c ^ 0xFFFFFFFFu;
}

static void write_header(uint8_t *slot, int format, int flags, int dtype, int component,
                         int d, int n_vec, uint32_t stored, uint64_t spill_off, uint32_t aux) {
  memset(slot, 0, HEADER_BYTES);
  slot[0] = 1;                                   /* format version */
  slot[1] = (uint8_t)format;
  slot[2] = (uint8_t)flags;
  slot[3] = (uint8_t)(dtype | (component << 4));
  put_u16(slot + 4, (uint16_t)d);
  put_u16(slot + 6, (uint16_t)n_vec);
  put_u32(slot + 8, (uint32_t)(n_vec * d * 2));  /* original length */
  put_u32(slot + 12, stored);
  put_u64(slot + 16, spill_off);
  put_u32(slot + 24, 0);                         /* CRC32: reserved */
  put_u32(slot + 28, aux);
}

/* the CRC32 of the stored bytes goes into the header (offset 24), with flag
 * bit 3 set; the spill offset is not covered, so it can be patched later */
static void set_crc(uint8_t *slot, const uint8_t *stored, size_t n) {
  slot[2] |= KVO_FLAG_CRC32;
  put_u32(slot + 24, kvo_crc32(stored, n));
}

int kvo_encode_segment(const uint16_t *vec, int dtype, int d, int n_vec, int heads,
                       int component, int codec, int is_protected,
                       float fixed_scale, uint64_t seed,
                       uint8_t *slot, uint8_t *spill, uint64_t spill_offset, int flags) {
  if (heads <= 0 || n_vec % heads) return -1;
  int eff = kvo_effective_codec(codec, d, n_vec, heads, is_protected);
  const int with_crc = flags & KVO_ENC_CRC32;
  size_t orig = (size_t)n_vec * (size_t)d * 2;
  size_t slot_bytes = kvo_slot_bytes(eff, d, n_vec, heads);
  memset(slot, 0, slot_bytes);
  if (eff == KVO_RAW) {
    write_header(slot, KVO_RAW, 1, dtype, component, d, n_vec, (uint32_t)orig, 0, 0);
    for (size_t i = 0; i < (size_t)n_vec * (size_t)d; i++) put_u16(slot + HEADER_BYTES + 2 * i, vec[i]);
    if (with_crc) set_crc(slot, slot + HEADER_BYTES, orig);
    return KVO_SEG_RAW_POLICY;
  }
  if (eff == KVO_ANS16) {
    /* lossless: no gate.  Kept only when slot plus the 256-byte aligned
     * payload saves 12.5% over the source; otherwise the segment stays raw
     * [OKV-SF "GPU ANS": incompressible pages remain raw]. */
    const size_t n = (size_t)n_vec * (size_t)d;
    uint8_t *pay = (uint8_t *)malloc(2 * (1024 + 2 * n));
    const size_t len = ans_encode_segment(vec, n, pay);
    const int keep = 8 * (slot_bytes + align_up(len, SLOT_ALIGN)) <= 7 * orig;
    if (keep) {
      write_header(slot, KVO_ANS16, FLAG_HEAP, dtype, component, d, n_vec, (uint32_t)len, spill_offset, 0);
      if (spill) {
        memcpy(spill, pay, len);
        if (with_crc) set_crc(slot, spill, len);
      }
    } else {
      write_header(slot, KVO_RAW, 2, dtype, component, d, n_vec, (uint32_t)orig, spill_offset, 0);
      if (spill) {
        for (size_t i = 0; i < n; i++) put_u16(spill + 2 * i, vec[i]);
        if (with_crc) set_crc(slot, spill, orig);
      }
    }
    free(pay);
    return keep ? KVO_SEG_ENCODED : KVO_SEG_RAW_DATA;
  }

  int bits = codec_bits(eff), cb = kvo_code_bytes(eff, d), mb = kvo_meta_bytes(eff);
  uint8_t *codes = slot + HEADER_BYTES;
  uint8_t *meta = codes + (size_t)n_vec * (size_t)cb;
  const size_t row = kvo_row_bytes(d, heads);     /* INT8_ROWS only */
  int8_t sigma[MAX_D];
  float cent[16], thr[15];
  if (eff == KVO_TQ3 || eff == KVO_TQ4) {
    kvo_signs(seed, d, sigma);
    kvo_codebook_f32(bits, cent, thr);
  }

  /* segment gate [OKV-SF "FP8 and TurboQuant"]: nonfinite values keep the
   * segment raw for every codec; FP8 codecs also for any |x| > 448 (source
   * value) instead of clipping. */
  int raw = 0;
  for (size_t i = 0; i < (size_t)n_vec * (size_t)d; i++) {
    float xv = src_to_f32(vec[i], dtype);
    if (!isfinite(xv)) raw = 1;
    if ((eff == KVO_FP8_DIRECT || eff == KVO_FP8_FIXED || eff == KVO_FP8_DYNAMIC) &&
        fabsf(xv) > 448.0f) raw = 1;
  }

  float x[MAX_D];
  for (int v = 0; v < n_vec && !raw; v++) {
    for (int i = 0; i < d; i++) x[i] = src_to_f32(vec[(size_t)v * d + i], dtype);
    uint8_t *cv = codes + (size_t)v * cb;
    uint8_t *mv = meta + (size_t)v * mb;
    if (eff == KVO_INT8_ROWS) {                   /* token t = v / heads, head h = v % heads */
      uint8_t *r = slot + ROWS_OFFSET + (size_t)(v / heads) * row;
      cv = r + (size_t)(v % heads) * (size_t)d;
      mv = r + (size_t)heads * (size_t)d + 2u * (size_t)(v % heads);
    }
    switch (eff) {
      case KVO_FP8_DIRECT: enc_fp8_direct(x, d, cv); break;
      case KVO_FP8_FIXED: enc_fp8_scaled(x, d, fixed_scale, cv); break;
      case KVO_FP8_DYNAMIC: {
        float s = fp8_dynamic_scale(x, d);
        put_u32(mv, f2u(s));
        enc_fp8_scaled(x, d, s, cv);
        break;
      }
      case KVO_INT8: {
        float s = int8_scale(x, d);
        put_u32(mv, f2u(s));
        enc_int8(x, d, s, cv);
        break;
      }
      case KVO_INT8_ROWS: {
        float s = int8_rows_scale(x, d);
        put_u16(mv, kvo_f32_to_bf16(s));
        enc_int8(x, d, s, cv);
        break;
      }
      case KVO_UNIFORM3: case KVO_UNIFORM4: raw |= enc_uniform(x, d, bits, cv, mv); break;
      case KVO_TQ3: case KVO_TQ4: raw |= enc_tq(x, d, bits, sigma, thr, cv, mv); break;
      default: return -1;
    }
  }

  if (raw) {
    memset(slot, 0, slot_bytes);
    write_header(slot, KVO_RAW, 2, dtype, component, d, n_vec, (uint32_t)orig, spill_offset, 0);
    if (spill) {
      for (size_t i = 0; i < (size_t)n_vec * (size_t)d; i++) put_u16(spill + 2 * i, vec[i]);
      if (with_crc) set_crc(slot, spill, orig);
    }
    return KVO_SEG_RAW_DATA;
  }
  /* the stored bytes: codes then metadata after the header, or for
   * INT8_ROWS the token rows at ROWS_OFFSET */
  const int rows = eff == KVO_INT8_ROWS;
  const size_t stored = rows ? (size_t)(n_vec / heads) * row : (size_t)n_vec * (cb + mb);
  write_header(slot, eff, 0, dtype, component, d, n_vec, (uint32_t)stored, 0,
               eff == KVO_FP8_FIXED ? f2u(fixed_scale) : 0);
  if (with_crc) set_crc(slot, slot + (rows ? ROWS_OFFSET : HEADER_BYTES), stored);
  return KVO_SEG_ENCODED;
}

int kvo_decode_segment(const uint8_t *slot, const uint8_t *buf_base,
                       int dtype, int d, int n_vec, int heads, uint64_t seed, uint16_t *out) {
  if (slot[0] != 1 || heads <= 0 || n_vec % heads) return -1;
  int format = slot[1], flags = slot[2];
  if ((slot[3] & 15) != dtype || get_u16(slot + 4) != d || get_u16(slot + 6) != n_vec) return -1;
  if (get_u32(slot + 8) != (uint32_t)(n_vec * d * 2)) return -1;
  size_t nel = (size_t)n_vec * (size_t)d;
  /* a CRC32, when present, is checked before anything is decoded */
  if (flags & KVO_FLAG_CRC32) {
    const uint8_t *stored = (flags & (2 | FLAG_HEAP)) ? buf_base + get_u64(slot + 16)
                            : slot + (format == KVO_INT8_ROWS ? ROWS_OFFSET : HEADER_BYTES);
    if ((flags & 2) && (flags & 4)) return -1;
    if (kvo_crc32(stored, get_u32(slot + 12)) != get_u32(slot + 24)) return -2;
  }
  if (flags & 2) {                                   /* raw, spilled */
    if (flags & 4) return -1;                        /* spill capacity was exhausted */
    const uint8_t *src = buf_base + get_u64(slot + 16);
    for (size_t i = 0; i < nel; i++) out[i] = get_u16(src + 2 * i);
    return 0;
  }
  if (format == KVO_RAW) {
    for (size_t i = 0; i < nel; i++) out[i] = get_u16(slot + HEADER_BYTES + 2 * i);
    return 0;
  }
  if (format == KVO_ANS16) {
    if (!(flags & FLAG_HEAP)) return -1;
    return ans_decode_segment(buf_base + get_u64(slot + 16), get_u32(slot + 12), nel, out) ? 0 : -1;
  }
  int bits = codec_bits(format), cb = kvo_code_bytes(format, d), mb = kvo_meta_bytes(format);
  const uint8_t *codes = slot + HEADER_BYTES;
  const uint8_t *meta = codes + (size_t)n_vec * cb;
  const size_t row = kvo_row_bytes(d, heads);
  int8_t sigma[MAX_D];
  float cent[16], thr[15];
  if (format == KVO_TQ3 || format == KVO_TQ4) {
    kvo_signs(seed, d, sigma);
    kvo_codebook_f32(bits, cent, thr);
  }
  float fixed = u2f(get_u32(slot + 28));
  for (int v = 0; v < n_vec; v++) {
    const uint8_t *cv = codes + (size_t)v * cb;
    const uint8_t *mv = meta + (size_t)v * mb;
    uint16_t *ov = out + (size_t)v * d;
    if (format == KVO_INT8_ROWS) {
      const uint8_t *r = slot + ROWS_OFFSET + (size_t)(v / heads) * row;
      cv = r + (size_t)(v % heads) * (size_t)d;
      mv = r + (size_t)heads * (size_t)d + 2u * (size_t)(v % heads);
    }
    switch (format) {
      case KVO_FP8_DIRECT:
        for (int i = 0; i < d; i++) ov[i] = f32_to_out(kvo_e4m3_to_f32(cv[i]), dtype);
        break;
      case KVO_FP8_FIXED: case KVO_FP8_DYNAMIC: {
        float s = format == KVO_FP8_FIXED ? fixed : u2f(get_u32(mv));
        for (int i = 0; i < d; i++) ov[i] = f32_to_out(kvo_e4m3_to_f32(cv[i]) * s, dtype);
        break;
      }
      case KVO_INT8: {
        float s = u2f(get_u32(mv));
        for (int i = 0; i < d; i++) ov[i] = f32_to_out((float)(int8_t)cv[i] * s, dtype);
        break;
      }
      case KVO_INT8_ROWS: {                        /* code x BF16 scale, rounded once */
        float s = kvo_bf16_to_f32(get_u16(mv));
        for (int i = 0; i < d; i++) ov[i] = f32_to_out((float)(int8_t)cv[i] * s, dtype);
        break;
      }
      case KVO_UNIFORM3: case KVO_UNIFORM4: dec_uniform(cv, mv, d, bits, dtype, ov); break;
      case KVO_TQ3: case KVO_TQ4: dec_tq(cv, mv, d, bits, sigma, cent, dtype, ov); break;
      default: return -1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the test harness (loops over the scalar definitions)    */
/* ------------------------------------------------------------------------ */
void kvo_f32_to_e4m3_n(const float *x, uint8_t *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_f32_to_e4m3(x[i]);
}
void kvo_e4m3_nearest_search_n(const float *x, uint8_t *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_e4m3_nearest_search(x[i]);
}
void kvo_e4m3_to_f32_n(const uint8_t *c, float *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_e4m3_to_f32(c[i]);
}
void kvo_f32_to_bf16_n(const float *x, uint16_t *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_f32_to_bf16(x[i]);
}
void kvo_f32_to_f16_n(const float *x, uint16_t *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_f32_to_f16(x[i]);
}
void kvo_f16_to_f32_n(const uint16_t *h, float *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = kvo_f16_to_f32(h[i]);
}
