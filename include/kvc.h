/*
 * kvc.h -- C ABI of libkvc: GPU encode/decode of paged KV-cache blocks on
 * AMD Instinct MI355X (gfx950), before offload and on restore.
 *
 * The operations are the ones described on these pages:
 *   [OKV-SF] OrbitKV docs, "KV precision and storage encoding":
 *            "FP8 and TurboQuant" (codecs, raw fallback, head dims, protected
 *            layers, payload sizes, layout validation for vLLM's packed
 *            [block, head, token, 2 x head_dim] layout and separate K/V
 *            tensors) and "Ownership, storage and GDS" (segment header:
 *            version, original length, format, stored length, CRC32; 12.5%
 *            keep rule; 16 MiB source cap; batched descriptor-based launches
 *            with statuses collected once per batch; retained arena;
 *            destinations validated for the whole request; teardown drains).
 *   [HIQ]    "Building a quantized HiCache for SGLang": "Building the INT8
 *            codec" (per-vector symmetric INT8) and "Integrating the codec"
 *            (the pool reports the encoded size per token).
 *   [KNLP]   "Asymmetric KV: methods and results": "Precision and scaling
 *            reference" (FP8 E4M3FN scale rule, fixed or per token/head).
 *
 * Conventions
 *  - All sizes are in bytes, all strides in elements.  Pointers are device
 *    pointers unless the comment says host.
 *  - Every call validates its arguments on the host first.  On any error it
 *    returns a nonzero kvc_status and has enqueued nothing and written
 *    nothing.
 *  - Encode/decode are asynchronous on the caller's HIP stream (never a host
 *    synchronisation, except to recycle the library's own small staging
 *    memory when more than a handful of calls are still in flight, or to
 *    release an offload-lane staging buffer after it has grown).  The
 *    caller owns the KV tensors, the page-id arrays, the encoded buffer and
 *    the descriptor array; the library owns only its arena.
 *  - A context may be used from one host thread at a time.
 *  - No C++ exception leaves the library: a failed host allocation returns
 *    KVC_E_NOMEM, from the call's checks and set-up, before it enqueues
 *    anything.
 *
 * Encoded format (version 1)
 *  Segment = (page, layer, component K or V) = T*H vectors of D elements, in
 *  canonical vector order v = token*H + head.  Segments of one call are laid
 *  out layer-major: s = ((layer * n_pages) + i) * 2 + component, each in its
 *  own slot at a deterministic offset (kvc_plan):
 *      slot = [32-B header][codes block: n_vec * code_bytes]
 *             [metadata block: n_vec * meta_bytes][zero padding to 256 B]
 *  Header (little-endian): u8 version=1, u8 format (codec of the stored
 *  bytes, KVC_RAW when raw), u8 flags (KVC_FLAG_*), u8 dtype | component<<4,
 *  u16 head_dim, u16 n_vec, u32 original_len, u32 stored_len,
 *  u64 spill_offset, u32 crc32, u32 aux (FP8_FIXED scale bits).
 *  crc32 (flag KVC_FLAG_CRC32, requested with KVC_CODEC_CRC32) is the CRC-32
 *  of zlib -- reflected polynomial 0xEDB88320, register preset to
 *  0xFFFFFFFF, result complemented -- of the stored_len stored bytes (the
 *  codes and metadata, or the raw bytes wherever they are kept) [OKV-SF
 *  "Ownership, storage and GDS": each segment carries a CRC32]; 0 without
 *  the flag.
 *  Codes are packed LSB-first (element i at bits [b*i, b*i+b) of the vector's
 *  code block); metadata per vector: FP32 scale (FP8_DYNAMIC, INT8), FP16 min
 *  + FP16 scale (UNIFORM*), FP16 norm (TQ*).
 *  KVC_INT8_ROWS lays its stored bytes out as records instead [HIQ "Why
 *  exactly 1,152 bytes?"]: from byte 128 of the slot (bytes 32..127 zero),
 *  one row per token: the INT8 codes of heads 0..H-1 (D bytes each), then
 *  their BF16 scales, then zeros to a multiple of 128 bytes (1,152 bytes at
 *  8 heads x 128).  Per vector: a = max(amax, BF16(1e-12)); scale =
 *  BF16(RN(a/127)); q = clamp(RNE(RN(x/scale)), +-127); decode rounds
 *  q*scale once to the output type.  stored_len = tokens * row bytes.
 *  KVC_ANS16 is lossless [OKV-SF "GPU ANS": typed 16-bit pages entropy coded,
 *  the exact output length checked on decompression, incompressible pages
 *  raw]: rANS (Duda 2013) over the low and the high byte plane of the
 *  segment's values in canonical order.  Each plane: a 16-byte header (u16
 *  mode, u16 K, zeros), then for mode 0 the raw n bytes, for mode 1 a 32-byte
 *  bitmap of the K symbols present, their u16 frequencies (summing to 4096:
 *  1 + floor(count * (4096 - K) / n) each, the remainder to the most
 *  frequent, lowest symbol on ties), 64 u16 stream lengths and the 64
 *  streams (element i in stream (i / 8) mod 64; state in [2^23, 2^31), byte
 *  renormalisation; a stream is [final state u32][renormalisation bytes,
 *  last emitted first]); zero padding to 16.  A plane is coded when that is
 *  shorter than raw.  The slot holds only the header (flag KVC_FLAG_HEAP);
 *  the payload goes to the spill region at spill_offset.  A segment whose
 *  256-byte slot plus 256-byte aligned payload does not save 12.5% is stored
 *  raw there (KVC_SEG_RAW_DATA); segments outside 4..32 KiB of source are raw
 *  by policy.
 *  A segment that must stay raw because of its data (a nonfinite value, an
 *  FP8 source value with |x| > 448, an FP16 metadata overflow) keeps its
 *  slot header (flags RAW_DATA) and its raw bytes go to the spill region of
 *  the output buffer (everything after the slot region), at spill_offset.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 2u
#define KVC_FORMAT_VERSION 1u
#define KVC_SLOT_ALIGN 256u
#define KVC_HEADER_BYTES 32u
#define KVC_MAX_SEGMENT_BYTES (16u << 20)
#define KVC_DEFAULT_WORKSPACE (64u << 20)

typedef struct kvc_ctx kvc_ctx;   /* opaque: one HIP device, its arena */

typedef enum {
  KVC_OK = 0,
  KVC_E_ARG = 1,          /* null pointer, bad enum, bad stride/alignment, bad scale */
  KVC_E_UNSUPPORTED = 2,  /* head_dim not in {32,64,128,256}, layout/dtype not supported */
  KVC_E_PAGE_RANGE = 3,   /* a page id outside [0, num_blocks) */
  KVC_E_DUP_DST = 4,      /* the same destination page twice in one decode */
  KVC_E_CAPACITY = 5,     /* output/input buffer smaller than the plan */
  KVC_E_BUDGET = 6,       /* per-call metadata exceeds the workspace budget */
  KVC_E_HIP = 7,          /* a HIP runtime call failed */
  KVC_E_NOMEM = 8         /* host memory for the call's bookkeeping ran out */
} kvc_status;

typedef enum { KVC_BF16 = 1, KVC_FP16 = 2 } kvc_dtype;

typedef enum {
  KVC_SEPARATE_NHD = 1,   /* per layer two tensors, K and V: [block][token][head][D] */
  KVC_PACKED_HT2D = 2     /* per layer one tensor (vLLM): [block][head][token][2*D], K then V */
} kvc_layout_kind;

/* Engine tensor geometry [OKV-SF "FP8 and TurboQuant": the packed and the
 * separate K/V layouts are validated explicitly; layout is never inferred
 * from byte counts].  Element (block b, token t, head h, dim i) of component
 * c is at  base_c + b*stride_block + t*stride_token + h*stride_head + i,
 * where base_K = k_base[l] and base_V = v_base[l] (separate) or
 * k_base[l] + head_dim (packed).  The innermost dimension is contiguous.
 * Requirements: base pointers 16-B aligned, strides positive multiples of 8
 * elements; SEPARATE_NHD: stride_head >= D, stride_token >= H*stride_head,
 * stride_block >= T*stride_token; PACKED_HT2D: stride_token >= 2*D,
 * stride_head >= T*stride_token, stride_block >= H*stride_head.  One page
 * of one layer must span fewer than 2^31 elements ((T-1)*stride_token +
 * (H-1)*stride_head + D, or + 2*D packed), else KVC_E_UNSUPPORTED. */
typedef struct {
  uint32_t abi;                 /* KVC_ABI_VERSION */
  uint32_t kind;                /* kvc_layout_kind */
  uint32_t dtype;               /* kvc_dtype */
  uint32_t layers, kv_heads, head_dim, tokens_per_page;
  uint32_t reserved;
  uint64_t num_blocks;          /* pages per layer tensor */
  int64_t stride_block, stride_token, stride_head;
  void *const *k_base;          /* host array [layers] of device pointers */
  void *const *v_base;          /* host array [layers]; NULL for PACKED_HT2D */
} kvc_layout;

typedef enum {
  KVC_RAW = 0,          /* stored unchanged */
  KVC_FP8_DIRECT = 1,   /* E4M3FN RNE cast, no scale [OKV-SF "FP8 and TurboQuant"] */
  KVC_FP8_FIXED = 2,    /* E4M3FN of RN(x/s), s per layer/component, clip +-448 [KNLP] */
  KVC_FP8_DYNAMIC = 3,  /* same with s = RN(max(amax,1e-12) * RN(1/448)) per vector [KNLP] */
  KVC_INT8 = 4,         /* s = RN(max(amax,1e-12)/127), q = RNE(RN(x/s)) clamp +-127 [HIQ] */
  KVC_UNIFORM3 = 5,     /* per-vector uniform 3-bit, FP16 min and scale [OKV-SF] */
  KVC_UNIFORM4 = 6,     /* per-vector uniform 4-bit, FP16 min and scale [OKV-SF] */
  KVC_TQ3 = 7,          /* TurboQuant MSE 3-bit + FP16 norm [OKV-SF] */
  KVC_TQ4 = 8,          /* TurboQuant MSE 4-bit + FP16 norm [OKV-SF] */
  KVC_INT8_ROWS = 9,    /* INT8 record: BF16 scales, 128-byte-padded token rows [HIQ] */
  KVC_ANS16 = 10        /* lossless rANS of the 16-bit values' byte planes [OKV-SF "GPU ANS"] */
} kvc_codec_id;

/* Codec choice per component.  fixed_scales: host array [layers][2] (K, V)
 * of FP32 scales, required iff a component uses KVC_FP8_FIXED (each must be
 * finite and in [2^-100, 2^100]).  protected_layers: host bitmap
 * [ceil(layers/8)] (bit l%8 of byte l/8), or NULL; protected layers are
 * stored raw [OKV-SF "FP8 and TurboQuant": some layers at the ends of each
 * pipeline stage are kept lossless; which ones is the caller's choice].  seed: rotation
 * seed of the TurboQuant sign generator (SplitMix64, version 1).  flags:
 * KVC_CODEC_CRC32 makes encode store each segment's CRC32 (KVC_FLAG_CRC32)
 * and makes decode verify it before it writes the page; a codec with a
 * KVC_ANS16 component requires it (else KVC_E_ARG), since a corrupted
 * entropy-coded stream shows only once it has been decoded; other bits and
 * `reserved` must be 0 (else KVC_E_ARG). */
#define KVC_CODEC_CRC32 1u
typedef struct {
  uint32_t k, v;                       /* kvc_codec_id */
  uint64_t seed;
  const float *fixed_scales;
  const uint8_t *protected_layers;
  uint32_t flags;                      /* KVC_CODEC_* */
  uint32_t reserved;
} kvc_codec;

/* Segment status, written by encode into kvc_segment_desc.status */
enum {
  KVC_SEG_ENCODED = 0,    /* stored with the requested codec */
  KVC_SEG_RAW_POLICY = 1, /* raw in its slot: protected layer, KVC_RAW, keep rule, size cap */
  KVC_SEG_RAW_DATA = 2,   /* raw because of its data, bytes in the spill region */
  KVC_SEG_CAPACITY = 3,   /* raw because of its data but the spill region was full: NOT stored */
  KVC_SEG_GUARD = 4       /* the kernel's own range check on its staged descriptor failed:
                             nothing was read or written for this segment (never expected) */
};
/* header / descriptor flags */
enum { KVC_FLAG_RAW_POLICY = 1, KVC_FLAG_RAW_DATA = 2, KVC_FLAG_CAPACITY = 4, KVC_FLAG_CRC32 = 8,
       KVC_FLAG_HEAP = 16 /* the stored bytes are at spill_offset (KVC_ANS16) */ };

/* One per segment, written by encode on the device (32 B).  Offsets are
 * relative to the start of the encode output buffer. */
typedef struct {
  uint64_t offset;        /* slot offset */
  uint64_t spill_offset;  /* raw bytes for KVC_SEG_RAW_DATA, else 0 */
  uint32_t stored_len;    /* payload bytes (codes + metadata, or raw bytes) */
  uint32_t original_len;  /* n_vec * D * element size */
  uint8_t version, format, flags, status;
  uint32_t crc32;         /* the header's crc32 (0 without KVC_FLAG_CRC32) */
} kvc_segment_desc;

/* Create a context on HIP device `hip_device` with a retained device arena
 * of `workspace_budget` bytes (0 = KVC_DEFAULT_WORKSPACE, the analogue of
 * OrbitKV's --storage-codec-budget default of 64 MB) holding per-call
 * descriptors and codebooks [OKV-SF "Ownership, storage and GDS"].
 * Errors: KVC_E_ARG (ctx NULL), KVC_E_HIP. */
kvc_status kvc_create(kvc_ctx **ctx, int hip_device, size_t workspace_budget);

/* Wait for all work the context launched, then free its memory
 * [OKV-SF: teardown drains GPU work before releasing memory].  NULL is a
 * no-op. */
kvc_status kvc_destroy(kvc_ctx *ctx);

/* Sizes for a call over n_pages pages (host only, no GPU needed):
 *  slot_bytes: bytes of the slot region (the output must be at least this);
 *  spill_bytes_suggested: a spill region for ~3% of the encodable segments
 *    (at least one segment) -- data-dependent raw segments beyond the spill
 *    capacity get KVC_SEG_CAPACITY;
 *  bytes_per_token: slot bytes per token of all layers, the encoded size a
 *    host pool reports [HIQ "Integrating the codec": get_size_per_token].
 * The CRC option changes no size (the CRC lives in the header).
 * Any output pointer may be NULL. */
kvc_status kvc_plan(const kvc_layout *layout, const kvc_codec *codec, uint32_t n_pages,
                    size_t *slot_bytes, size_t *spill_bytes_suggested,
                    size_t *bytes_per_token);

/* Host-only validation used by kvc_encode_pages (exposed so callers and
 * tests can check arguments without a GPU).  page_ids: host [n_pages]. */
kvc_status kvc_validate_encode(const kvc_layout *layout, const kvc_codec *codec,
                               const int32_t *page_ids, uint32_t n_pages, size_t out_bytes);
/* Same for kvc_decode_pages; also rejects duplicate destination pages. */
kvc_status kvc_validate_decode(const kvc_layout *layout, const kvc_codec *codec,
                               const int32_t *dst_page_ids, uint32_t n_pages, size_t in_bytes);

/* Encode the pages page_ids (host [n_pages], source block ids) of every
 * layer into `out` (device, out_bytes >= slot_bytes; the remainder is the
 * spill region).  desc (device, [layers*n_pages*2]) receives one
 * descriptor per segment.  Everything is enqueued on `stream` (hipStream_t,
 * NULL = default stream).  Segments are independent: one launch covers the
 * whole call, and the caller reads the statuses once per batch. */
kvc_status kvc_encode_pages(kvc_ctx *ctx, const kvc_layout *layout, const kvc_codec *codec,
                            const int32_t *page_ids, uint32_t n_pages,
                            void *out, size_t out_bytes, kvc_segment_desc *desc,
                            void *stream);

/* Decode a buffer produced by kvc_encode_pages with the same layout
 * geometry, codec and n_pages into the destination pages dst_page_ids (host
 * [n_pages], distinct, validated for the whole request before anything is
 * enqueued [OKV-SF "Ownership, storage and GDS"]).  Raw segments are copied
 * bit-exactly.  seg_status (device [layers*n_pages*2] u8, may be NULL)
 * receives 0 per decoded segment, 1 when the slot header does not match
 * the geometry/codec (including its stored length and whether it carries a
 * CRC32, which must agree with codec->flags) or the segment was not stored
 * (KVC_SEG_CAPACITY), 2 when the kernel's range check on its staged
 * descriptor failed, or 3 when the stored bytes do not match the header's
 * CRC32 (KVC_CODEC_CRC32 only); in cases 1-3 the destination page is left
 * unchanged, with one exception: a KVC_ANS16 payload that matches its CRC32
 * and whose headers, model, stream lengths, padding and exact length all
 * check out, but one of whose streams does not decode to exactly its length
 * in the initial state (or starts outside the state interval) -- bytes the
 * encoder never writes -- reports 1 after its page has been written.
 * Enqueued on `stream`. */
kvc_status kvc_decode_pages(kvc_ctx *ctx, const kvc_layout *layout, const kvc_codec *codec,
                            const void *in, size_t in_bytes,
                            const int32_t *dst_page_ids, uint32_t n_pages,
                            uint8_t *seg_status, void *stream);

/* Decode only the segments of layers [layer_begin, layer_end) of a buffer
 * produced by kvc_encode_pages (same arguments otherwise, and the same
 * in_bytes) -- the per-layer step of a layer-by-layer restore [HIQ
 * "Integrating the codec": load_to_device_per_layer].  Segment statuses
 * land at their usual indices of seg_status.  KVC_E_ARG if layer_end <
 * layer_begin or layer_end > layers; an empty range enqueues nothing. */
kvc_status kvc_decode_layers(kvc_ctx *ctx, const kvc_layout *layout, const kvc_codec *codec,
                             const void *in, size_t in_bytes,
                             const int32_t *dst_page_ids, uint32_t n_pages,
                             uint32_t layer_begin, uint32_t layer_end,
                             uint8_t *seg_status, void *stream);

/* Offload lane, device to host [HIQ "Integrating the codec": GPU staging
 * buffers, separate for backup and restoration, grown when necessary and
 * never replaced while a stream still uses them].
 * Encode the pages page_ids of every layer into the context's offload
 * staging buffer, always with a CRC32 per segment (KVC_CODEC_CRC32 is added
 * to codec->flags) [OKV-SF "Ownership, storage and GDS": every stored
 * segment carries a CRC32 that is checked before decode], then copy the
 * slot region and the layers*n_pages*2 descriptors to host_out and
 * host_desc, and of the spill region (the rest of host_bytes) only the bytes
 * the encode used, all enqueued on `stream`.  The used size is read back
 * from the device once per call [OKV-SF "Ownership, storage and GDS": sizes
 * are collected once per batch]: the call waits for the encode to finish
 * (not for the copies) and stores in *host_used (may be NULL) the bytes of
 * host_out that hold the encoding -- the slot region plus the used spill
 * bytes; a restore needs only those.  host_out and host_desc must be pinned
 * host memory (hipHostMalloc, or a pinned torch tensor); they are written
 * when the stream reaches the copies and must stay allocated until then.
 * The bytes in host_out[0, *host_used) are what kvc_encode_pages with
 * KVC_CODEC_CRC32 writes to a device buffer of host_bytes bytes.
 * Errors as kvc_validate_encode (host_bytes in place of out_bytes), and
 * KVC_E_ARG for memory that is not pinned host memory.  The staging buffer
 * grows to host_bytes + the descriptors; a buffer it replaces is freed once
 * the work queued on it has finished (freeing may wait for the device). */
kvc_status kvc_offload_pages(kvc_ctx *ctx, const kvc_layout *layout, const kvc_codec *codec,
                             const int32_t *page_ids, uint32_t n_pages,
                             void *host_out, size_t host_bytes, kvc_segment_desc *host_desc,
                             size_t *host_used, void *stream);

/* Offload lane, host to device: restore layers [layer_begin, layer_end) of
 * an encoded buffer held in pinned host memory (host_in, in_bytes: what
 * kvc_offload_pages wrote -- in_bytes may be its *host_used -- or any
 * kvc_encode_pages output made with KVC_CODEC_CRC32 and copied to host;
 * the lane always checks the CRC32, as if codec->flags held KVC_CODEC_CRC32)
 * into the destination pages dst_page_ids (host [n_pages], distinct, all
 * validated before anything is enqueued).  The context's restore staging
 * buffer receives the spill region, then each layer's slots, on an internal
 * copy stream that starts after the work already queued on `stream`; layer
 * l is decoded on `stream` as soon as its bytes have arrived, so copies of
 * later layers overlap decodes of earlier ones.  After layer l's decode,
 * layer_ready[l - layer_begin] (a hipEvent_t, may be NULL; the array may be
 * NULL) is recorded on `stream`: copy, decode and scatter of the layer all
 * precede it [HIQ "Making asynchronous restoration safe"].  seg_status as
 * in kvc_decode_pages.  host_in must stay allocated and unchanged until the
 * stream passes this call.  Errors as kvc_validate_decode, KVC_E_ARG for a
 * bad layer range or memory that is not pinned host memory. */
kvc_status kvc_restore_pages(kvc_ctx *ctx, const kvc_layout *layout, const kvc_codec *codec,
                             const void *host_in, size_t in_bytes,
                             const int32_t *dst_page_ids, uint32_t n_pages,
                             uint32_t layer_begin, uint32_t layer_end,
                             uint8_t *seg_status, void *const *layer_ready, void *stream);

/* Allocation-free variant of kvc_encode_pages, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  No context: the per-call side table,
 * page ids and spill cursor live in a fixed device array of this library,
 * one copy per GPU held until the process ends (about 350 KiB: the codec
 * tables, a 256-byte cursor, 2 x 256 side-table entries of 32 bytes and
 * 65,536 page ids).  The call allocates nothing: no hipMalloc, hipFree, host
 * heap or pinned memory.  The first call on a device looks the array up and
 * copies the codec tables into it (a synchronous copy): make that call
 * outside any graph capture.
 * Arguments, output bytes, descriptors and errors are those of
 * kvc_encode_pages on the current HIP device, plus KVC_E_BUDGET when
 * layout->layers > 256 or n_pages > 65536.  The side table and the zeroed
 * spill cursor are copied from the call's stack with a pageable copy, which
 * HIP completes before returning (it may wait for earlier work on the
 * stream); page_ids (host) is copied the same way when it is pageable, and
 * must stay unchanged until the stream passes this call when it is pinned.
 * Every call on a GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from several host threads) race and give
 * undefined results; calls ordered on one stream are safe. */
kvc_status kvc_encode_pages_noalloc(const kvc_layout *layout, const kvc_codec *codec,
                                    const int32_t *page_ids, uint32_t n_pages,
                                    void *out, size_t out_bytes, kvc_segment_desc *desc,
                                    void *stream);

/* Short text for a status code (static storage). */
const char *kvc_status_string(kvc_status s);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
