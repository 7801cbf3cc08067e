// kvc_internal.h -- structures shared by the host half of libkvc and its
// gfx950 kernels.  Not part of the public ABI (include/kvc.h is).
#pragma once
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "kvc.h"

namespace kvc {

// One workgroup per segment: one wave (64 threads) for segments of at most
// kSmallSegmentBytes source bytes -- a small segment would leave a larger
// workgroup with little data in flight per wave, while one-wave workgroups
// keep up to 32 segments in flight per CU -- else kEncodeThreads for encode
// (two waves: the compute-heavy TurboQuant encode keeps more vectors in
// flight per wave; a large call without CRC32 whose components all encode
// raw, FP8 or INT8 keeps one wave) and kDecodeThreads for decode (four
// waves; one at D = 256 without CRC32).
constexpr int kEncodeThreads = 128;
// encode with the CRC option above kSmallSegmentBytes: two waves as well
// (the 1 KiB of nibble tables leaves occupancy as it is; four waves would
// give each wave fewer vectors but nearly as many CRC rounds)
constexpr int kEncodeThreadsCrc = 128;
constexpr int kDecodeThreads = 256;
constexpr int kThreadsSmall = 64;
constexpr uint32_t kSmallSegmentBytes = 16384;

// A head vector of D elements is held by a group of lanes_per_vector(D)
// lanes; a workgroup of nt threads holds groups_per_workgroup(D, nt)
// groups, and group g handles vectors g, g + GW, g + 2*GW, ... of a segment
// (GW = groups per workgroup).
constexpr int lanes_per_vector(int d) { return d == 32 ? 2 : (d == 64 ? 4 : (d == 128 ? 8 : 16)); }
constexpr int groups_per_workgroup(int d, int nt) { return nt / lanes_per_vector(d); }
// vectors per group whose loads are in flight together (one batch)
constexpr int kBatchVectors = 2;
constexpr uint64_t kSlotAlign = KVC_SLOT_ALIGN;
constexpr uint32_t kHeaderBytes = KVC_HEADER_BYTES;

// INT8 record codec (KVC_INT8_ROWS): one row per token holding its heads'
// codes and their BF16 scales, padded to a multiple of 128 bytes; the rows
// start kRowsOffset bytes into the slot.
constexpr uint32_t kRowsOffset = 128;
constexpr uint32_t row_bytes(uint32_t d, uint32_t heads) { return (heads * d + 2 * heads + 127) / 128 * 128; }

// Bucketize table for TurboQuant encode: cell c of the real line,
// c = RNE(kCellScale * z) + kCellOffset, holds the one threshold that may lie
// inside the cell (or +inf) and the count of thresholds below the cell, so
// that #{k : B_k < z} = base + (z > T).  kCellScale = 4 makes every cell
// (width 1/4) narrower than the closest pair of 3- or 4-bit thresholds.
constexpr float kCellScale = 4.0f;
constexpr int kCellOffset = 64;               // |z| <= sqrt(256) = 16 -> |4z| <= 64
constexpr int kCells = 2 * kCellOffset + 1;   // 129

constexpr uint32_t kMaxStageBytes = 32768;    // LDS staging limit per workgroup

struct CellEntry {
  float thr;
  uint32_t base;
};

// CRC-32 tables (reflected polynomial 0xEDB88320) for the CRC of a byte
// range computed by all N = 64 * 2^w lanes of a workgroup (w = 0, 1, 2 for
// 64, 128, 256 threads): lane j takes 16-byte units j, j + N, j + 2N, ...
// and steps its register over each 4-byte word with nibble tables (eight
// lookups of 16 entries per word, by linearity of the CRC register update);
// the last word of a unit that has a successor in the same lane uses tj[w],
// which also carries the register over the 16 (N - 1) bytes that the other
// lanes take in between.  Each lane then carries its register r over the
// 16 (N - 1 - j) bytes after its last unit: the product r * s_j modulo the
// polynomial with s_j = x^(8 * 16 (N - 1 - j)), formed as the xor of
// x^i * s_j over the coefficients i set in r (the powers pw*, grouped four
// to a 16-byte load: pw[i / 4][j][i % 4]; the decode kernels read only s_j
// and multiply it by x between the steps), and the lanes' registers are
// xored.  Registers are in the reflected order: bit 31 holds the
// coefficient of x^0.
constexpr int kCrcLanes = 64;               // lanes of a wave
constexpr int kCrcLaneSets = 3;             // N = 64, 128, 256
constexpr int kCrcLevels = 8;               // log2 of the largest N
struct CrcTables {
  uint32_t t[8][16];                        // register after a word whose only nonzero nibble k is v, from a zero register
  uint32_t tj[kCrcLaneSets][8][16];         // t[k][v] carried over 16 (64 * 2^w - 1) more zero bytes
  uint32_t pw64[8][64][4];                  // x^i * s_j mod P for N = 64, 128, 256
  uint32_t pw128[8][128][4];
  uint32_t pw256[8][256][4];
  // lv[b][k][v]: the register v << 4k carried over 16 * 2^b zero bytes, i.e.
  // multiplied by x^(128 * 2^b) mod P (a pairwise combination of lanes)
  uint32_t lv[kCrcLevels][8][16];
};
static_assert(sizeof(CrcTables) % 16 == 0, "CRC tables are copied in 16-byte units");
// the part of CrcTables one kernel keeps in LDS: t and its lane count's tj
struct CrcLds {
  uint32_t t[8][16];
  uint32_t tj[8][16];
};

// Reciprocals of the rANS encoder (KVC_ANS16), indexed by the frequency f in
// [1, 4096]: ceil(2^(31+l) / f) with l = ceil(log2 f) for f >= 2, so that
// floor(x / f) = (x * rcp) >> (31 + l) for every x < 2^31 (Granlund and
// Montgomery, PLDI 1994, Thm 4.2); 2^32 - 1 for f = 1.
constexpr uint32_t kAnsRcpEntries = 4100;

// Per-ctx constant tables (device, in the arena).
struct Tables {
  CellEntry cells[2][kCells];                 // [0]: 3-bit, [1]: 4-bit
  float centroids[2][16];
  alignas(16) CrcTables crc;
  uint32_t ans_rcp[kAnsRcpEntries];
};

// Per-(layer, component) entry of a call (device, in the arena), indexed by
// 2*layer + component.  Every field sits at a fixed, naturally aligned offset
// of a 32-byte record, so the kernels read it with aligned scalar loads.
struct SideEntry {
  const uint16_t* base;                       // element 0 of block 0 of this component
  uint64_t slot_base;                         // slot offset of (layer, page 0, component)
  uint32_t page_stride;                       // slot bytes of one page of the layer (K + V)
  uint32_t slot_bytes;                        // slot size of this component's segments
  uint32_t codec;                             // effective codec (KVC_RAW for policy raw)
  float fixed;                                // FP8_FIXED scale
};
static_assert(sizeof(SideEntry) == 32, "SideEntry is a 32-byte record");

// the largest call whose side table and page ids ride in the kernel arguments
constexpr uint32_t kInlineSides = 16;         // 2 * layers
constexpr uint32_t kInlinePages = 256;
// Spill cursors of such calls: a pool of 8-byte slots in the context's
// arena, zero when the context is created and never reset; call k uses slot
// k mod kCursorSlots and tags its value with the lap k / kCursorSlots + 1
// (bits 40..63), so the first reservation of a call starts from zero
// whatever an earlier call left in the slot.  Offsets use bits 0..39.
constexpr uint32_t kCursorSlots = 65536;
constexpr int kCursorLapShift = 40;

struct CallParams {
  const SideEntry* sides;                     // [2 * n_layers]
  const int32_t* pages;                       // source (encode) / destination (decode) block ids
  const Tables* tables;
  uint8_t* buf;                               // encode output / decode input
  uint64_t buf_bytes;
  uint64_t slot_region;                       // spill region = [slot_region, buf_bytes)
  kvc_segment_desc* desc;                     // encode: descriptors (device)
  uint8_t* seg_status;                        // decode: statuses (device, may be null)
  unsigned long long* spill_cursor;           // encode: bytes used in the spill region
  uint32_t cursor_lap;                        // 0: spill_cursor starts at zero; else its lap tag
  uint64_t base_lo, base_hi;                  // range of every layer base pointer (guard)
  int64_t sb, st, sh;                         // element strides
  uint64_t heads_magic;                       // ceil(2^32 / heads): t = (v * magic) >> 32 = v / heads
  uint32_t threads;                           // threads per workgroup (see with_threads in the host)
  // Walking a lane from vector v to v + GW (GW = groups_per_workgroup(D, threads)):
  // head h -> h + walk_dh (minus heads on wrap), element offset within the
  // page -> + walk_step (+ walk_wrap on wrap); all modulo 2^32.  A page spans
  // fewer than 2^31 elements, so every offset actually used is exact.
  uint32_t st32, sh32;                        // stride_token, stride_head
  uint32_t walk_dh, walk_step, walk_wrap;
  // Nonzero when vector v of a page starts at element v * D (stride_head = D,
  // stride_token = heads * D) and the vectors fill whole batches of every
  // group (heads * tokens a multiple of GW * kBatchVectors): the batches per
  // group, which the fixed-size codec loops then walk without the head
  // counter or per-vector bounds.  0 otherwise.
  uint32_t linear_iters;
  // Encode: bytes of dynamic LDS in which each coded (non-raw) segment's slot
  // is assembled before it is written out with full-line stores; 0 when
  // some coded slot exceeds kMaxStageBytes (then codes go straight out).
  uint32_t stage_bytes;
  // 1: encode stores each segment's CRC32, decode verifies it; the CRC
  // tables then sit in dynamic LDS right after the staging bytes.
  uint32_t crc;
  // First segment of the launch: a launch covers the segments [seg_base,
  // seg_base + workgroups) of the call (a range of whole layers).
  uint32_t seg_base;
  uint32_t n_pages, n_layers, heads, tokens;
  uint32_t row_bytes;                         // KVC_INT8_ROWS: bytes of one token row
  uint32_t dtype;                             // kvc_dtype
  uint32_t num_blocks;                        // page ids must be below this (guard)
  uint32_t sign_mask[8];                      // TurboQuant signs, bit i = (sigma_i < 0)
  // Small calls: the side table and the page ids travel in the kernel
  // arguments (inline_tables = 1), so nothing is uploaded before the launch
  uint32_t inline_tables;
  SideEntry sides_inline[kInlineSides];
  int32_t pages_inline[kInlinePages];
};

// Allocation-free encode (kvc_encode_pages_noalloc): every call on a GPU
// uses that GPU's copy of one file-scope device array (kvc_kernels.hip),
// laid out as [Tables | spill cursor (256 B) | side table | page ids], for
// calls of at most kNoAllocMaxLayers layers and kNoAllocMaxPages pages.
constexpr uint32_t kNoAllocMaxLayers = 256;
constexpr uint32_t kNoAllocMaxPages = 65536;
constexpr size_t kNoAllocCursorOff = (sizeof(Tables) + 255) / 256 * 256;
constexpr size_t kNoAllocSidesOff = kNoAllocCursorOff + 256;
constexpr size_t kNoAllocPagesOff = kNoAllocSidesOff + sizeof(SideEntry) * 2 * kNoAllocMaxLayers;
constexpr size_t kNoAllocScratchBytes = kNoAllocPagesOff + sizeof(int32_t) * kNoAllocMaxPages;
constexpr int kNoAllocMaxDevices = 64;
// Device address of the current device's scratch array (`device` must be
// current).  The first call for a device looks the address up and copies
// host_tables into its head; later calls return the kept address.
hipError_t noalloc_scratch(int device, const Tables* host_tables, uint8_t** ptr);

// Launchers (kvc_kernels.hip): segments [p.seg_base, p.seg_base +
// n_segments).  Return hipSuccess or the launch error.
hipError_t launch_encode(const CallParams& p, uint32_t head_dim, uint64_t n_segments,
                         hipStream_t stream);
hipError_t launch_decode(const CallParams& p, uint32_t head_dim, uint64_t n_segments,
                         hipStream_t stream);
// The entropy stage (KVC_ANS16 segments; the kernels above skip them), one
// wave per segment, over the same segments.  Encode: p.stage_bytes (at
// least n + 16 for n values per segment) of LDS hold one coded byte plane.
hipError_t launch_ans_encode(const CallParams& p, uint32_t head_dim, uint64_t n_segments, hipStream_t stream);
hipError_t launch_ans_decode(const CallParams& p, uint32_t head_dim, uint64_t n_segments, hipStream_t stream);
// ANS16 applies to segments of this many source bytes (others stay raw)
constexpr uint32_t kAnsMinBytes = 4096, kAnsMaxBytes = 32768;

}  // namespace kvc
