/*
 * kvc_oracle.h -- plain, slow, scalar CPU oracle for the paged KV-cache codecs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library never
 * links, includes or calls anything in this directory, and this directory
 * shares no source with it.
 *
 * Sources (the pages):
 *   [OKV-SF]  OrbitKV docs, "KV precision and storage encoding",
 *             sections "FP8 and TurboQuant", "Ownership, storage and GDS"
 *             and "GPU ANS".
 *   [HIQ]     "Building a quantized HiCache for SGLang", sections
 *             "Building the INT8 codec" and "Why exactly 1,152 bytes?".
 *   [KNLP]    knlp, "Asymmetric KV: methods and results", section
 *             "Precision and scaling reference".
 *
 * Every floating-point step is one IEEE binary32 operation with
 * round-to-nearest-even (RN), no contraction (build with -ffp-contract=off),
 * correctly rounded divide and sqrt.  Conversions to BF16/FP16/E4M3FN are
 * written from the formats' definitions (nearest representable value, ties to
 * the even significand), not from any hardware instruction.
 *
 * Pins (tests/test_oracle_pins.py): E4M3FN/BF16/FP16 conversions against
 * brute-force search and library casts over every source pattern; the FP8
 * scale constants; the INT8 worked example and ties-to-even; Lloyd-Max
 * tables, distortion and optimality conditions; SplitMix64's published
 * vector; the WHT against the Hadamard matrix and its involution; payload
 * sizes; closed-form TurboQuant codes of signed Hadamard rows; nearest-level
 * and nearest-centroid brute force; gate cases; the INT8 record's sizes
 * (tests/golden/int8_record_sizes.json), a worked token row, the closed form
 * of power-of-two scales and its error bound; the ANS16 model normalisation
 * invariants, lossless round trips, the closed form of a constant plane, the
 * raw-plane rule, the coded size against the model's cross-entropy (both
 * bounds) and the rejection of streams that end early, run long or start
 * outside the state interval.
 *
 * Parity unpinned (by the pages): the exact bits of TurboQuant codes at
 * threshold boundaries and of TurboQuant decodes depend on the FP32
 * operation order chosen here (normalise by RN(1/n) with the FP32 norm,
 * pairwise sum-of-squares tree, WHT stages in ascending span, decode
 * g = RN(n_h / RN(RN(sqrt(q)) * RN(sqrt(D))))); the pages fix only the
 * steps, so only the invariants above pin them.  The uniform codec's
 * codes are the plain binary32 quotient RN(RN(x - m_h) / sigma_h) rounded
 * to the nearest integer, pinned against an exact-rational construction of
 * that definition and the tie cases it decides.  The ANS16
 * payload bytes follow this library's own format (the pages name nvCOMP's
 * ANS without giving its format): its pins fix what any such coder must
 * satisfy (lossless, sizes near the entropy, exact-length checks), not the
 * byte layout itself.
 */
#ifndef KVC_ORACLE_H
#define KVC_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* codec ids == format byte of the encoded segment */
enum {
  KVO_RAW = 0, KVO_FP8_DIRECT = 1, KVO_FP8_FIXED = 2, KVO_FP8_DYNAMIC = 3,
  KVO_INT8 = 4, KVO_UNIFORM3 = 5, KVO_UNIFORM4 = 6, KVO_TQ3 = 7, KVO_TQ4 = 8,
  KVO_INT8_ROWS = 9,  /* INT8 with BF16 scales in 128-byte-padded token rows */
  KVO_ANS16 = 10      /* lossless rANS of the low and high byte planes */
};
enum { KVO_BF16 = 1, KVO_FP16 = 2 };
/* segment status returned by the encoder */
enum { KVO_SEG_ENCODED = 0, KVO_SEG_RAW_POLICY = 1, KVO_SEG_RAW_DATA = 2 };
/* encode option: compute a CRC32 of the stored bytes; header flag bit 3 */
enum { KVO_ENC_CRC32 = 1, KVO_FLAG_CRC32 = 8 };
/* header flag bit 4: the stored bytes sit at spill_offset (ANS16 payloads) */
enum { KVO_FLAG_HEAP = 16 };

/* ---- lossless entropy stage (ANS16) ----
 * Frequencies summing to 4096 from 256 counts over n symbols. */
void   kvo_ans_normalize(const uint32_t *count, uint32_t n, uint16_t *freq);
/* One byte plane of n symbols: 64 interleaved rANS streams, or the raw
 * bytes when that is shorter; returns the serialised size (a multiple of
 * 16).  out: at least 1024 + 2n bytes. */
size_t kvo_ans_encode_plane(const uint8_t *sym, size_t n, uint8_t *out);
/* Size of the rANS body of n <= 16384 symbols (0 beyond), coded or not. */
size_t kvo_ans_coded_body(const uint8_t *sym, size_t n);
/* Inverse; returns the bytes consumed, 0 on any inconsistency (bad table,
 * stream overrun, a stream not ending exactly at its length in the initial
 * state). */
size_t kvo_ans_decode_plane(const uint8_t *in, size_t avail, size_t n, uint8_t *sym);

/* CRC-32 (reflected polynomial 0xEDB88320, preset and final complement) */
uint32_t kvo_crc32(const uint8_t *p, size_t n);

/* ---- number formats (bit-level definitions) ---- */
float    kvo_bf16_to_f32(uint16_t h);
float    kvo_f16_to_f32(uint16_t h);
uint16_t kvo_f32_to_bf16(float x);        /* RNE, overflow -> Inf, NaN kept NaN */
uint16_t kvo_f32_to_f16(float x);         /* RNE, overflow -> Inf, NaN kept NaN */
uint8_t  kvo_f32_to_e4m3(float x);        /* RNE; |x| must be <= 448 or NaN     */
float    kvo_e4m3_to_f32(uint8_t c);
/* nearest-value search over all 254 finite E4M3FN codes (brute force, used
 * only to pin kvo_f32_to_e4m3) */
uint8_t  kvo_e4m3_nearest_search(float x);

/* ---- method constants ---- */
/* Lloyd-Max quantizer of N(0,1) with 2^bits levels, computed in double by the
 * alternating centroid / midpoint conditions until a fixed point.  Writes
 * 2^bits centroids (ascending) and 2^bits-1 thresholds (midpoints), both in
 * double.  Returns the number of iterations used. */
int  kvo_lloyd_max(int bits, double *centroids, double *thresholds);
/* FP32 codebook of the format: C_k = RN(c_k), B_k = RN((c_{k-1}+c_k)/2). */
void kvo_codebook_f32(int bits, float *centroids, float *thresholds);
/* Deterministic signs, generator version 1: sigma_i = -1 iff bit 63 of the
 * i-th SplitMix64 output (state initialised to seed) is set. */
void kvo_signs(uint64_t seed, int d, int8_t *sigma);
uint64_t kvo_splitmix64_next(uint64_t *state);

/* ---- per-vector codecs (x are source bits, one vector of D elements) ---- */
/* Walsh-Hadamard transform, unnormalised Sylvester order, in place, stages
 * h = 1, 2, 4, ..., d/2, each (a, b) -> (RN(a+b), RN(a-b)). */
void kvo_wht_f32(float *v, int d);
/* Pairwise sum of squares: leaves RN(x_i^2), adjacent pairs first. */
float kvo_sumsq_tree(const float *x, int d);

/* ---- format sizes ---- */
int    kvo_code_bytes(int codec, int d);   /* code bytes per vector        */
int    kvo_meta_bytes(int codec);          /* metadata bytes per vector    */
/* aligned slot incl. header; heads = vectors per token (n_vec = tokens *
 * heads), which only the INT8_ROWS layout depends on */
size_t kvo_slot_bytes(int codec, int d, int n_vec, int heads);
/* INT8_ROWS: bytes of one token row, heads*d codes + heads BF16 scales
 * padded to a multiple of 128 */
size_t kvo_row_bytes(int d, int heads);
/* codec actually used for a segment after the static rules (RAW policy,
 * 12.5% keep rule, 16 MiB cap) */
int    kvo_effective_codec(int codec, int d, int n_vec, int heads, int is_protected);

/* ---- segments ----
 * vec: n_vec*d source bit patterns in canonical vector order (v = t*H + h),
 * heads = H (n_vec must be a multiple of it).
 * slot: kvo_slot_bytes(effective codec) bytes, fully written (header, payload,
 * zero padding).  INT8_ROWS stores, from byte 128 of the slot, one row per
 * token: its H vectors' codes (h-major), its H BF16 scales, zero padding to
 * kvo_row_bytes; every other codec stores the codes block then the metadata
 * block right after the 32-byte header.  ANS16 writes only the header into
 * the slot (flag KVO_FLAG_HEAP) and its payload -- plane 0 then plane 1 --
 * into spill, at spill_offset; an ANS16 segment whose slot plus 256-byte
 * aligned payload would not save 12.5% is stored raw (KVO_SEG_RAW_DATA).  For a data-dependent RAW segment the slot carries only the
 * header (payload zero) and the raw bytes go to spill (n_vec*d*2 bytes, if
 * spill != NULL); spill_offset is written into the header.  flags:
 * KVO_ENC_CRC32 stores the CRC32 of the stored bytes (the payload, or the raw
 * bytes in the slot or the spill) in the header.
 * Returns KVO_SEG_*. */
int kvo_encode_segment(const uint16_t *vec, int dtype, int d, int n_vec, int heads,
                       int component, int codec, int is_protected,
                       float fixed_scale, uint64_t seed,
                       uint8_t *slot, uint8_t *spill, uint64_t spill_offset, int flags);
/* Decode one slot into n_vec*d output bit patterns (canonical order).
 * buf_base is the start of the buffer the spill offsets refer to.
 * Returns 0 on success, -1 on a malformed header, -2 when the segment
 * carries a CRC32 that its stored bytes do not match. */
int kvo_decode_segment(const uint8_t *slot, const uint8_t *buf_base,
                       int dtype, int d, int n_vec, int heads, uint64_t seed,
                       uint16_t *out);

/* array loops over the scalar conversions, for the test harness */
void kvo_f32_to_e4m3_n(const float *x, uint8_t *out, size_t n);
void kvo_e4m3_nearest_search_n(const float *x, uint8_t *out, size_t n);
void kvo_e4m3_to_f32_n(const uint8_t *c, float *out, size_t n);
void kvo_f32_to_bf16_n(const float *x, uint16_t *out, size_t n);
void kvo_f32_to_f16_n(const float *x, uint16_t *out, size_t n);
void kvo_f16_to_f32_n(const uint16_t *h, float *out, size_t n);

#ifdef __cplusplus
}
#endif
#endif
