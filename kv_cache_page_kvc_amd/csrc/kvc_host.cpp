// kvc_host.cpp -- host half of libkvc: argument validation, the slot plan,
// the retained device arena, format constants (Lloyd-Max codebook, sign
// generator) and the launches.
//
// Behaviour follows OrbitKV docs, "KV precision and storage encoding":
//  "FP8 and TurboQuant": layouts and K/V roles are validated explicitly;
//    head dims 32/64/128/256; protected layers stay exact; the sign
//    generator is versioned and seeded.
//  "Ownership, storage and GDS": keep an encoded segment only when its
//    aligned footprint saves >= 12.5%; sources up to 16 MiB are encoded;
//    one descriptor-driven launch per batch with statuses collected once;
//    a retained arena bounded by the workspace budget; restore validates
//    destinations for the whole request first; teardown drains GPU work.
// and "Building a quantized HiCache for SGLang", "Integrating the codec":
//    the encoded size per token is reported for capacity accounting; the
//    offload and restore directions have their own persistent GPU staging
//    buffers, grown when needed and never freed while a stream still uses
//    them; copy, decode and scatter of a restored layer are ordered before
//    the layer is signalled ready.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <vector>

#include "kvc.h"
#include "kvc_internal.h"

using namespace kvc;

struct kvc_ctx {
  int device = 0;
  size_t budget = 0;
  uint8_t* arena = nullptr;          // device: [Tables | ring]
  uint8_t* staging = nullptr;        // pinned host mirror of the ring
  size_t ring_begin = 0, ring_end = 0, head = 0;
  uint64_t small_encodes = 0;        // encode calls whose spill cursor is a pool slot
  struct InFlight {
    size_t off, size;
    hipEvent_t ev;
  };
  std::vector<InFlight> inflight;
  std::vector<hipEvent_t> free_events;
  // Device staging of the offload lane, one per direction (0: offload, 1:
  // restore), so transfers in the two directions never share bytes.  `last`
  // is recorded after the last use of `ptr`; the next call on any stream
  // waits for it before reusing the buffer.
  struct Staging {
    uint8_t* ptr = nullptr;
    size_t cap = 0;
    hipEvent_t last = nullptr;
  };
  Staging lane[2];
  // buffers replaced by a larger one, freed once their last use has finished
  struct Retired {
    uint8_t* ptr;
    hipEvent_t ev;
  };
  std::vector<Retired> retired;
  hipStream_t copy_stream = nullptr;   // restore: host-to-device copies, ahead of the decodes
  hipEvent_t fork = nullptr;           // restore: orders the copy stream after the caller's work
  std::vector<hipEvent_t> layer_copied;
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------ formats
int codec_bits(int c) {
  switch (c) {
    case KVC_UNIFORM3: case KVC_TQ3: return 3;
    case KVC_UNIFORM4: case KVC_TQ4: return 4;
    case KVC_RAW: return 16;
    default: return 8;
  }
}
int codec_meta(int c) {
  switch (c) {
    case KVC_FP8_DYNAMIC: case KVC_INT8: case KVC_UNIFORM3: case KVC_UNIFORM4: return 4;
    case KVC_TQ3: case KVC_TQ4: return 2;
    default: return 0;
  }
}
// heads: vectors per token (n_vec = tokens * heads); only the record codec's
// slot depends on it
uint64_t slot_size(int codec, uint32_t d, uint32_t n_vec, uint32_t heads) {
  if (codec == KVC_ANS16) return align_up(KVC_HEADER_BYTES, KVC_SLOT_ALIGN);   // payload in the spill region
  if (codec == KVC_INT8_ROWS)
    return align_up(kRowsOffset + (uint64_t)(n_vec / heads) * row_bytes(d, heads), KVC_SLOT_ALIGN);
  const uint64_t per_vec = (uint64_t)codec_bits(codec) * d / 8 + (uint64_t)codec_meta(codec);
  return align_up(KVC_HEADER_BYTES + per_vec * n_vec, KVC_SLOT_ALIGN);
}
// codec used after the static rules: raw for protected layers and KVC_RAW,
// raw for sources above 16 MiB, raw if the aligned slot saves < 12.5%.
int effective_codec(int codec, uint32_t d, uint32_t n_vec, uint32_t heads, bool prot) {
  const uint64_t orig = (uint64_t)n_vec * d * 2;
  if (prot || codec == KVC_RAW) return KVC_RAW;
  if (orig > KVC_MAX_SEGMENT_BYTES) return KVC_RAW;
  if (codec == KVC_ANS16 && (orig < kAnsMinBytes || orig > kAnsMaxBytes)) return KVC_RAW;
  if (8 * slot_size(codec, d, n_vec, heads) > 7 * orig) return KVC_RAW;
  return codec;
}
bool is_protected(const kvc_codec* c, uint32_t l) {
  return c->protected_layers && ((c->protected_layers[l >> 3] >> (l & 7)) & 1);
}

// ------------------------------------------------------------------ constants
// Gaussian Lloyd-Max quantizer with n levels, by alternating the two
// optimality conditions (cell boundaries at midpoints, levels at the
// conditional means of their cells) until nothing moves.
double phi(double x) { return std::exp(-0.5 * x * x) * 0.3989422804014326779399461; }
double upper(double x) { return 0.5 * std::erfc(x * 0.7071067811865475244008444); }
// P(lo < X < hi), accurate in both tails
double cell_mass(double lo, double hi) {
  if (lo >= 0) return upper(lo) - upper(hi);
  if (hi <= 0) return upper(-hi) - upper(-lo);
  return 1.0 - upper(hi) - upper(-lo);
}
constexpr int kMaxLevels = 16;
void lloyd_max(int n, double* lev) {           // n <= kMaxLevels
  for (int k = 0; k < n; k++) lev[k] = -3.0 + 6.0 * (k + 0.5) / n;
  double b[kMaxLevels + 1];
  for (int it = 0; it < 4000000; it++) {
    b[0] = -INFINITY;
    b[n] = INFINITY;
    for (int k = 1; k < n; k++) b[k] = 0.5 * (lev[k - 1] + lev[k]);
    double moved = 0.0;
    for (int k = 0; k < n; k++) {
      const double num = (std::isinf(b[k]) ? 0.0 : phi(b[k])) - (std::isinf(b[k + 1]) ? 0.0 : phi(b[k + 1]));
      const double m = num / cell_mass(b[k], b[k + 1]);
      moved = std::max(moved, std::fabs(m - lev[k]));
      lev[k] = m;
    }
    if (moved < 1e-15) break;
  }
  for (int k = 0; k < n / 2; k++) {            // exact symmetry
    const double a = 0.5 * (lev[n - 1 - k] - lev[k]);
    lev[k] = -a;
    lev[n - 1 - k] = a;
  }
}

// CRC-32 tables (zlib's CRC: reflected polynomial 0xEDB88320), built from
// the bitwise definition; see CrcTables for how the kernels use them.
void build_crc_tables(CrcTables& c) {
  uint32_t byte_tab[256];
  for (uint32_t b = 0; b < 256; b++) {
    uint32_t r = b;
    for (int i = 0; i < 8; i++) r = (r >> 1) ^ (0xEDB88320u & (0u - (r & 1u)));
    byte_tab[b] = r;
  }
  auto zero_byte = [&byte_tab](uint32_t r) { return (r >> 8) ^ byte_tab[r & 0xFF]; };
  // register after the four bytes of x from a zero register, then `zeros` zero bytes
  auto word_then_zeros = [&](uint32_t x, uint32_t zeros) {
    uint32_t r = x;
    for (int b = 0; b < 4; b++) r = zero_byte(r);
    for (uint32_t i = 0; i < zeros; i++) r = zero_byte(r);
    return r;
  };
  for (int k = 0; k < 8; k++)
    for (uint32_t v = 0; v < 16; v++) c.t[k][v] = word_then_zeros(v << (4 * k), 0);
  for (int w = 0; w < kCrcLaneSets; w++) {
    const uint32_t lanes = (uint32_t)kCrcLanes << w;
    for (int k = 0; k < 8; k++)
      for (uint32_t v = 0; v < 16; v++) c.tj[w][k][v] = word_then_zeros(v << (4 * k), 16u * (lanes - 1));
    uint32_t* pw = w == 0 ? &c.pw64[0][0][0] : (w == 1 ? &c.pw128[0][0][0] : &c.pw256[0][0][0]);
    uint32_t s = 0x80000000u;                  // x^0: s_j for the last lane, then one unit more per lane
    for (uint32_t j = lanes; j-- > 0;) {
      uint32_t xi = s;                         // x^i * s_j
      for (uint32_t i = 0; i < 32; i++) {
        pw[((i / 4) * lanes + j) * 4 + i % 4] = xi;
        xi = (xi >> 1) ^ (0xEDB88320u & (0u - (xi & 1u)));   // times x
      }
      for (int b = 0; b < 16; b++) s = zero_byte(s);
    }
  }
  for (int lvl = 0; lvl < kCrcLevels; lvl++)
    for (int k = 0; k < 8; k++)
      for (uint32_t v = 0; v < 16; v++) {
        uint32_t r = v << (4 * k);
        for (uint32_t i = 0; i < (16u << lvl); i++) r = zero_byte(r);
        c.lv[lvl][k][v] = r;
      }
}

void build_tables(Tables& t) {
  build_crc_tables(t.crc);
  std::memset(t.ans_rcp, 0, sizeof(t.ans_rcp));
  t.ans_rcp[1] = 0xFFFFFFFFu;
  for (uint32_t f = 2; f <= 4096; f++) {
    uint32_t l = 0;
    while ((1u << l) < f) l++;
    t.ans_rcp[f] = (uint32_t)((((uint64_t)1 << (31 + l)) + f - 1) / f);
  }
  for (int which = 0; which < 2; which++) {
    const int bits = which ? 4 : 3, n = 1 << bits;
    double lev[kMaxLevels];
    lloyd_max(n, lev);
    float thr[15];
    for (int k = 0; k < n; k++) t.centroids[which][k] = (float)lev[k];
    for (int k = 0; k < n - 1; k++) thr[k] = (float)(0.5 * (lev[k] + lev[k + 1]));
    // cells: c = RNE(4 z) + 64, i.e. 4z in [c-64-0.5, c-64+0.5].  Every
    // threshold lies well inside (-15.875, 15.875): the edge cells hold none,
    // which lets the encoder clamp z to +-16 without changing a code.
    for (int c = 0; c < kCells; c++) {
      const double lo = (c - kCellOffset - 0.5) / kCellScale, hi = (c - kCellOffset + 0.5) / kCellScale;
      uint32_t below = 0;
      int inside = -1;
      for (int k = 0; k < n - 1; k++) {
        if ((double)thr[k] < lo) below++;
        else if ((double)thr[k] <= hi) inside = k;
      }
      t.cells[which][c].thr = inside >= 0 ? thr[inside] : INFINITY;
      t.cells[which][c].base = below;
    }
  }
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014); sign generator version 1:
// sigma_i = -1 iff bit 63 of the i-th output from state = seed.
void sign_mask(uint64_t seed, uint32_t d, uint32_t mask[8]) {
  std::memset(mask, 0, 8 * sizeof(uint32_t));
  uint64_t state = seed;
  for (uint32_t i = 0; i < d; i++) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    if (z >> 63) mask[i >> 5] |= 1u << (i & 31);
  }
}

// ------------------------------------------------------------------ validation
kvc_status check_layout(const kvc_layout* L) {
  if (!L || L->abi != KVC_ABI_VERSION) return KVC_E_ARG;
  if (L->dtype != KVC_BF16 && L->dtype != KVC_FP16) return KVC_E_UNSUPPORTED;
  if (L->kind != KVC_SEPARATE_NHD && L->kind != KVC_PACKED_HT2D) return KVC_E_UNSUPPORTED;
  const uint32_t D = L->head_dim;
  if (D != 32 && D != 64 && D != 128 && D != 256) return KVC_E_UNSUPPORTED;
  if (L->layers == 0 || L->kv_heads == 0 || L->tokens_per_page == 0 || L->num_blocks == 0) return KVC_E_ARG;
  const uint64_t n_vec = (uint64_t)L->kv_heads * L->tokens_per_page;
  if (n_vec > 65535) return KVC_E_UNSUPPORTED;                 // header field is 16 bits
  if (L->num_blocks > (uint64_t)std::numeric_limits<int32_t>::max()) return KVC_E_ARG;
  const int64_t sb = L->stride_block, st = L->stride_token, sh = L->stride_head;
  if (sb <= 0 || st <= 0 || sh <= 0 || (sb % 8) || (st % 8) || (sh % 8)) return KVC_E_ARG;
  const int64_t H = L->kv_heads, T = L->tokens_per_page;
  if (L->kind == KVC_SEPARATE_NHD) {
    if (sh < (int64_t)D || st < H * sh || sb < T * st) return KVC_E_ARG;
    if (!L->v_base) return KVC_E_ARG;
  } else {
    if (st < 2 * (int64_t)D || sh < T * st || sb < H * sh) return KVC_E_ARG;
    if (L->v_base) return KVC_E_ARG;
  }
  // the kernels address a page's elements with 32-bit offsets
  const int64_t page_extent = (T - 1) * st + (H - 1) * sh + (L->kind == KVC_SEPARATE_NHD ? 1 : 2) * (int64_t)D;
  if (page_extent >= (int64_t)1 << 31) return KVC_E_UNSUPPORTED;
  if (!L->k_base) return KVC_E_ARG;
  for (uint32_t l = 0; l < L->layers; l++) {
    const void* k = L->k_base[l];
    if (!k || ((uintptr_t)k & 15)) return KVC_E_ARG;
    if (L->kind == KVC_SEPARATE_NHD) {
      const void* v = L->v_base[l];
      if (!v || ((uintptr_t)v & 15)) return KVC_E_ARG;
    }
  }
  return KVC_OK;
}

kvc_status check_codec(const kvc_layout* L, const kvc_codec* c) {
  if (!c || c->k > KVC_ANS16 || c->v > KVC_ANS16) return KVC_E_ARG;
  if ((c->flags & ~KVC_CODEC_CRC32) || c->reserved) return KVC_E_ARG;
  // the entropy decoder can tell a corrupted stream only once it has
  // written the page: the segment CRC32 rejects it before
  if ((c->k == KVC_ANS16 || c->v == KVC_ANS16) && !(c->flags & KVC_CODEC_CRC32)) return KVC_E_ARG;
  if (c->k == KVC_FP8_FIXED || c->v == KVC_FP8_FIXED) {
    if (!c->fixed_scales) return KVC_E_ARG;
    for (uint32_t l = 0; l < L->layers; l++)
      for (int comp = 0; comp < 2; comp++) {
        if ((comp ? c->v : c->k) != KVC_FP8_FIXED) continue;
        const float s = c->fixed_scales[2 * l + comp];
        if (!(s >= 0x1p-100f && s <= 0x1p100f)) return KVC_E_ARG;   // also rejects NaN
      }
  }
  return KVC_OK;
}

// The slot plan of a call: per layer its slot offset and, per component,
// its slot size and effective codec.  The per-layer arrays live in storage
// the caller provides (HeapPlan: vectors; the allocation-free entry point:
// fixed arrays on its stack).
struct Plan {
  uint64_t* layer_off = nullptr;
  uint32_t* slot[2] = {nullptr, nullptr};
  uint8_t* eff[2] = {nullptr, nullptr};
  uint64_t total = 0;
  uint64_t per_page = 0;      // slot bytes of one page over all layers
  uint64_t encodable = 0;     // segments not raw by policy
  uint64_t ans = 0;           // of which KVC_ANS16 (payload in the spill region)
  bool light = true;          // every component raw, FP8 (direct, dynamic or fixed), INT8 or
                              // ANS16: no TurboQuant, uniform or record arithmetic in encode
};

// Fill p (whose arrays hold at least L->layers entries).
void fill_plan(const kvc_layout* L, const kvc_codec* c, uint32_t n_pages, Plan& p) {
  const uint32_t n_vec = L->kv_heads * L->tokens_per_page;
  p.total = p.per_page = p.encodable = p.ans = 0;
  p.light = true;
  uint64_t off = 0;
  for (uint32_t l = 0; l < L->layers; l++) {
    const bool prot = is_protected(c, l);
    uint64_t page = 0;
    for (int comp = 0; comp < 2; comp++) {
      const int e = effective_codec(comp ? c->v : c->k, L->head_dim, n_vec, L->kv_heads, prot);
      const uint32_t sz = (uint32_t)slot_size(e, L->head_dim, n_vec, L->kv_heads);
      if (p.eff[comp]) p.eff[comp][l] = (uint8_t)e;
      if (p.slot[comp]) p.slot[comp][l] = sz;
      page += sz;
      if (e != KVC_RAW) p.encodable += n_pages;
      if (e == KVC_ANS16) p.ans += n_pages;
      if (e != KVC_RAW && e != KVC_FP8_DIRECT && e != KVC_FP8_DYNAMIC && e != KVC_FP8_FIXED && e != KVC_INT8 &&
          e != KVC_ANS16)
        p.light = false;
    }
    if (p.layer_off) p.layer_off[l] = off;
    p.per_page += page;
    off += page * n_pages;
  }
  p.total = off;
}

// A plan with the per-layer arrays on the heap (not copyable: the pointers
// refer to its own vectors).
struct HeapPlan : Plan {
  std::vector<uint64_t> lo;
  std::vector<uint32_t> sz[2];
  std::vector<uint8_t> ef[2];
  HeapPlan(const kvc_layout* L, const kvc_codec* c, uint32_t n_pages)
      : lo(L->layers), sz{std::vector<uint32_t>(L->layers), std::vector<uint32_t>(L->layers)},
        ef{std::vector<uint8_t>(L->layers), std::vector<uint8_t>(L->layers)} {
    layer_off = lo.data();
    for (int comp = 0; comp < 2; comp++) {
      slot[comp] = sz[comp].data();
      eff[comp] = ef[comp].data();
    }
    fill_plan(L, c, n_pages, *this);
  }
  HeapPlan(const HeapPlan&) = delete;
  HeapPlan& operator=(const HeapPlan&) = delete;
};

// the plan's totals only (no per-layer arrays)
Plan plan_totals(const kvc_layout* L, const kvc_codec* c, uint32_t n_pages) {
  Plan p;
  fill_plan(L, c, n_pages, p);
  return p;
}

kvc_status check_pages(const kvc_layout* L, const int32_t* ids, uint32_t n, bool distinct) {
  if (n == 0) return KVC_OK;
  if (!ids) return KVC_E_ARG;
  for (uint32_t i = 0; i < n; i++)
    if (ids[i] < 0 || (uint64_t)ids[i] >= L->num_blocks) return KVC_E_PAGE_RANGE;
  if (distinct) {
    std::vector<int32_t> s(ids, ids + n);
    std::sort(s.begin(), s.end());
    if (std::adjacent_find(s.begin(), s.end()) != s.end()) return KVC_E_DUP_DST;
  }
  return KVC_OK;
}

kvc_status check_grid(const kvc_layout* L, uint32_t n) {
  const uint64_t nseg = (uint64_t)L->layers * n * 2;
  return nseg > 0x7FFFFFFFull ? KVC_E_ARG : KVC_OK;
}

// per-call metadata in the arena: [SideEntry x 2L][page ids][spill cursor]
size_t call_bytes(uint32_t layers, uint32_t n) {
  return align_up(sizeof(SideEntry) * 2 * layers, kAlign) + align_up(sizeof(int32_t) * (size_t)n, kAlign) + kAlign;
}

size_t tables_bytes() { return align_up(sizeof(Tables), kAlign); }
// arena: [Tables | spill-cursor pool of small encode calls | ring]
size_t cursor_pool_offset() { return tables_bytes(); }
size_t cursor_pool_bytes() { return align_up(sizeof(unsigned long long) * kCursorSlots, kAlign); }

struct DeviceGuard {
  int old = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old) != hipSuccess) old = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (old >= 0) (void)hipSetDevice(old);
  }
};

// reserve `size` bytes of the ring; waits only for calls whose metadata
// occupies the bytes about to be reused
kvc_status ring_alloc(kvc_ctx* ctx, size_t size, size_t* off) {
  if (size > ctx->ring_end - ctx->ring_begin) return KVC_E_BUDGET;
  // room for every event this call may retire and for ring_commit's entry,
  // so that no container grows (or throws) once work is enqueued
  ctx->free_events.reserve(ctx->free_events.size() + ctx->inflight.size());
  ctx->inflight.reserve(ctx->inflight.size() + 1);
  // retire finished calls
  for (size_t i = 0; i < ctx->inflight.size();) {
    if (hipEventQuery(ctx->inflight[i].ev) == hipSuccess) {
      ctx->free_events.push_back(ctx->inflight[i].ev);
      ctx->inflight.erase(ctx->inflight.begin() + (long)i);
    } else {
      i++;
    }
  }
  if (ctx->head + size > ctx->ring_end) ctx->head = ctx->ring_begin;
  const size_t a = ctx->head, b = ctx->head + size;
  for (size_t i = 0; i < ctx->inflight.size();) {
    const auto& f = ctx->inflight[i];
    if (f.off < b && a < f.off + f.size) {
      if (hipEventSynchronize(f.ev) != hipSuccess) return KVC_E_HIP;
      ctx->free_events.push_back(f.ev);
      ctx->inflight.erase(ctx->inflight.begin() + (long)i);
    } else {
      i++;
    }
  }
  *off = a;
  ctx->head = b;
  return KVC_OK;
}

kvc_status ring_commit(kvc_ctx* ctx, size_t off, size_t size, hipStream_t stream) {
  if (size == 0) return KVC_OK;                 // the call took no ring bytes
  hipEvent_t ev;
  if (!ctx->free_events.empty()) {
    ev = ctx->free_events.back();
    ctx->free_events.pop_back();
  } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    return KVC_E_HIP;
  }
  if (hipEventRecord(ev, stream) != hipSuccess) return KVC_E_HIP;
  ctx->inflight.push_back({off, size, ev});
  return KVC_OK;
}

hipEvent_t new_event() {
  hipEvent_t e = nullptr;
  return hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess ? e : nullptr;
}

// free the retired staging buffers whose last use has finished (all of them
// when `wait`)
void reap_retired(kvc_ctx* ctx, bool wait) {
  for (size_t i = 0; i < ctx->retired.size();) {
    auto& r = ctx->retired[i];
    const bool done = !r.ev || (wait ? hipEventSynchronize(r.ev) == hipSuccess : hipEventQuery(r.ev) == hipSuccess);
    if (done || wait) {
      (void)hipFree(r.ptr);
      if (r.ev) (void)hipEventDestroy(r.ev);
      ctx->retired.erase(ctx->retired.begin() + (long)i);
    } else {
      i++;
    }
  }
}

// Make lane `dir` hold at least `bytes`.  A smaller buffer is retired with
// its last-use event and freed only after that event has completed, so work
// still queued on it keeps valid memory; the new buffer starts with no use.
kvc_status lane_reserve(kvc_ctx* ctx, int dir, size_t bytes) {
  reap_retired(ctx, false);
  auto& st = ctx->lane[dir];
  if (st.cap >= bytes) return KVC_OK;
  const size_t cap = align_up(std::max(bytes, st.cap + st.cap / 4), 1u << 20);
  ctx->retired.reserve(ctx->retired.size() + 1);      // before the buffer exists
  uint8_t* p = nullptr;
  if (hipMalloc(&p, cap) != hipSuccess) return KVC_E_HIP;
  if (st.ptr) ctx->retired.push_back({st.ptr, st.last});
  else if (st.last) (void)hipEventDestroy(st.last);
  st.ptr = p;
  st.cap = cap;
  st.last = new_event();
  return st.last ? KVC_OK : KVC_E_HIP;
}

// host memory that the copy engines can reach without a bounce (allocated
// with hipHostMalloc, as torch's pinned tensors are): both ends of the range.
// A failed query sets the runtime's last error; it is cleared here so that
// the caller's next error check does not report it.
bool pinned_range(const void* p, size_t n) {
  unsigned int f = 0;
  if (!p || n == 0) return false;
  const bool ok = hipHostGetFlags(&f, const_cast<void*>(p)) == hipSuccess &&
                  hipHostGetFlags(&f, static_cast<uint8_t*>(const_cast<void*>(p)) + n - 1) == hipSuccess;
  if (!ok) (void)hipGetLastError();
  return ok;
}

// The call's side table (into se, 2 * layers entries) and every field of P
// but the device pointers (sides, pages, spill_cursor, tables, buf, desc,
// seg_status) and the buffer sizes.
void fill_call(const kvc_layout* L, const kvc_codec* c, const Plan& plan, uint32_t n, SideEntry* se, CallParams* P) {
  uint64_t lo = ~0ull, hi = 0;
  uint32_t stage = 0;
  for (uint32_t l = 0; l < L->layers; l++) {
    const uint16_t* bases[2] = {
        static_cast<const uint16_t*>(L->k_base[l]),
        L->kind == KVC_PACKED_HT2D ? static_cast<const uint16_t*>(L->k_base[l]) + L->head_dim
                                   : static_cast<const uint16_t*>(L->v_base[l])};
    for (int comp = 0; comp < 2; comp++) {
      SideEntry e{};
      e.base = bases[comp];
      e.slot_base = plan.layer_off[l] + (comp ? plan.slot[0][l] : 0u);
      e.page_stride = plan.slot[0][l] + plan.slot[1][l];
      e.slot_bytes = plan.slot[comp][l];
      e.codec = plan.eff[comp][l];
      e.fixed = c->fixed_scales ? c->fixed_scales[2 * l + comp] : 1.0f;
      se[2 * l + comp] = e;
      if (e.codec != KVC_RAW) stage = std::max<uint32_t>(stage, e.slot_bytes);
      lo = std::min<uint64_t>(lo, (uint64_t)(uintptr_t)e.base);
      hi = std::max<uint64_t>(hi, (uint64_t)(uintptr_t)e.base);
    }
  }
  P->base_lo = lo;
  P->base_hi = hi;
  P->stage_bytes = stage <= kMaxStageBytes ? stage : 0;   // slot sizes are multiples of 256
  P->num_blocks = (uint32_t)L->num_blocks;
  P->sb = L->stride_block;
  P->st = L->stride_token;
  P->sh = L->stride_head;
  P->n_pages = n;
  P->n_layers = L->layers;
  P->heads = L->kv_heads;
  // exact for every vector index v < 2^16 because heads <= 2^16 (v * heads < 2^32)
  P->heads_magic = ((1ull << 32) + L->kv_heads - 1) / L->kv_heads;
  {
    const uint32_t H = L->kv_heads;
    const uint32_t st = (uint32_t)L->stride_token, sh = (uint32_t)L->stride_head;   // < 2^31 (check_layout)
    P->st32 = st;
    P->sh32 = sh;
    P->walk_wrap = st - H * sh;                         // modulo 2^32
    // the workgroup size and its walk constants are set per launch (with_threads)
    P->threads = 0;
  }
  P->tokens = L->tokens_per_page;
  P->row_bytes = row_bytes(L->head_dim, L->kv_heads);
  P->dtype = L->dtype;
  P->crc = (c->flags & KVC_CODEC_CRC32) ? 1u : 0u;
  sign_mask(c->seed, L->head_dim, P->sign_mask);
}

// Stage the call's layer table, page ids and zeroed spill cursor (encode
// only: cursor = true), fill params.  A small call (at most kInlineSides
// side entries and kInlinePages pages) carries its table and page ids in the
// kernel arguments; only an encode's cursor then takes ring bytes, zeroed by
// a one-thread kernel.  Larger calls stage everything in the context's ring
// and upload it in one copy.  ring_size is 0 when no ring bytes were taken.
kvc_status stage_call(kvc_ctx* ctx, const kvc_layout* L, const kvc_codec* c, const Plan& plan,
                      const int32_t* pages, uint32_t n, hipStream_t stream, CallParams* P, size_t* ring_off,
                      size_t* ring_size, bool cursor) {
  *ring_off = 0;
  *ring_size = 0;
  P->tables = reinterpret_cast<const Tables*>(ctx->arena);
  if (2 * L->layers <= kInlineSides && n <= kInlinePages) {
    fill_call(L, c, plan, n, P->sides_inline, P);
    std::memcpy(P->pages_inline, pages, sizeof(int32_t) * (size_t)n);
    P->inline_tables = 1;
    P->sides = nullptr;
    P->pages = nullptr;
    P->spill_cursor = nullptr;
    P->cursor_lap = 0;
    if (!cursor) return KVC_OK;
    // a pool slot tagged with this call's lap: no upload, no clearing launch
    const uint64_t k = ctx->small_encodes++;
    P->spill_cursor = reinterpret_cast<unsigned long long*>(ctx->arena + cursor_pool_offset()) + k % kCursorSlots;
    P->cursor_lap = (uint32_t)((k / kCursorSlots) % ((1u << (64 - kCursorLapShift)) - 1u)) + 1u;
    return KVC_OK;
  }
  const size_t need = call_bytes(L->layers, n);
  size_t off = 0;
  kvc_status st = ring_alloc(ctx, need, &off);
  if (st != KVC_OK) return st;
  uint8_t* h = ctx->staging + off;
  fill_call(L, c, plan, n, reinterpret_cast<SideEntry*>(h), P);
  P->inline_tables = 0;
  const size_t pages_off = align_up(sizeof(SideEntry) * 2 * L->layers, kAlign);
  std::memcpy(h + pages_off, pages, sizeof(int32_t) * (size_t)n);
  const size_t cur_off = pages_off + align_up(sizeof(int32_t) * (size_t)n, kAlign);
  std::memset(h + cur_off, 0, kAlign);
  if (hipMemcpyAsync(ctx->arena + off, h, need, hipMemcpyHostToDevice, stream) != hipSuccess) return KVC_E_HIP;
  uint8_t* d = ctx->arena + off;
  P->sides = reinterpret_cast<const SideEntry*>(d);
  P->pages = reinterpret_cast<const int32_t*>(d + pages_off);
  P->spill_cursor = reinterpret_cast<unsigned long long*>(d + cur_off);
  *ring_off = off;
  *ring_size = need;
  return KVC_OK;
}

// Encode / decode launches of a call: the fixed-size codecs' kernel (not
// when every segment is KVC_ANS16), then, when some component uses
// KVC_ANS16, the entropy stage's kernel over the same segments (each skips
// the other's segments).  The entropy encode assembles one coded byte plane
// at a time in LDS: at most n + 16 bytes for n values per segment.
bool all_ans(const kvc_layout* L, const Plan& plan, const CallParams& P) {
  return plan.ans == 2ull * L->layers * P.n_pages;
}
// P for workgroups of nt threads: a lane walks from vector v to v + GW with
// GW = groups_per_workgroup(D, nt): head + walk_dh (minus H on wrap), element
// offset + walk_step (+ walk_wrap on wrap), all modulo 2^32
CallParams with_threads(const CallParams& P, const kvc_layout* L, uint32_t nt) {
  CallParams W = P;
  const uint32_t H = L->kv_heads, gw = (uint32_t)groups_per_workgroup((int)L->head_dim, (int)nt);
  W.threads = nt;
  W.walk_dh = gw % H;
  W.walk_step = (gw / H) * P.st32 + (gw % H) * P.sh32;
  const uint32_t n_vec = H * L->tokens_per_page, batch = gw * (uint32_t)kBatchVectors;
  W.linear_iters = P.sh32 == L->head_dim && P.st32 == H * L->head_dim && n_vec % batch == 0 ? n_vec / batch : 0;
  return W;
}
// one wave for small segments, else the direction's workgroup size
uint32_t workgroup_threads(const kvc_layout* L, uint32_t big) {
  const uint32_t seg_bytes = L->kv_heads * L->tokens_per_page * L->head_dim * 2;
  return seg_bytes <= kSmallSegmentBytes ? (uint32_t)kThreadsSmall : big;
}
// Encode: a call without CRC32 whose components all encode with little
// arithmetic per element (raw, FP8 direct, dynamic or fixed, INT8) runs one
// wave per segment at every size when it has segments enough to keep 32 in
// flight on each of 256 CUs -- more segments in flight per CU; the others
// run two waves above kSmallSegmentBytes.  With CRC32 one wave measured
// 7-16% slower for these calls (one wave's 64 lanes take twice the rounds
// over the slot that two waves take).
constexpr uint64_t kLightOneWaveSegments = 32 * 256;
hipError_t run_encode(const CallParams& P, const kvc_layout* L, const Plan& plan, uint64_t nseg, hipStream_t s) {
  const uint32_t nt = plan.light && !P.crc && nseg >= kLightOneWaveSegments
                          ? (uint32_t)kThreadsSmall
                          : workgroup_threads(L, P.crc ? kEncodeThreadsCrc : kEncodeThreads);
  hipError_t e = all_ans(L, plan, P) ? hipSuccess : launch_encode(with_threads(P, L, nt), L->head_dim, nseg, s);
  if (e == hipSuccess && plan.ans) {
    CallParams A = P;
    A.stage_bytes = L->kv_heads * L->tokens_per_page * L->head_dim + 16;
    e = launch_ans_encode(A, L->head_dim, nseg, s);
  }
  return e;
}
// Decode: four waves above kSmallSegmentBytes, but one wave at D = 256
// without CRC32, which measured 3-4% faster there (16-lane groups: four
// waves give each group only four vectors of a segment)
hipError_t run_decode(const CallParams& P, const kvc_layout* L, const Plan& plan, uint64_t nseg, hipStream_t s) {
  const uint32_t nt =
      L->head_dim == 256 && !P.crc ? (uint32_t)kThreadsSmall : workgroup_threads(L, kDecodeThreads);
  hipError_t e = all_ans(L, plan, P) ? hipSuccess : launch_decode(with_threads(P, L, nt), L->head_dim, nseg, s);
  if (e == hipSuccess && plan.ans) e = launch_ans_decode(P, L->head_dim, nseg, s);
  return e;
}

// Host containers can throw std::bad_alloc; no exception crosses the C ABI.
template <class F>
kvc_status no_throw(F&& f) noexcept {
  try {
    return f();
  } catch (...) {
    return KVC_E_NOMEM;
  }
}

// Tables for the allocation-free entry point, built once per process into
// static storage (no heap).
const Tables* static_tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] { build_tables(t); });
  return &t;
}

}  // namespace

extern "C" {

const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_ARG: return "invalid argument";
    case KVC_E_UNSUPPORTED: return "unsupported geometry";
    case KVC_E_PAGE_RANGE: return "page id out of range";
    case KVC_E_DUP_DST: return "duplicate destination page";
    case KVC_E_CAPACITY: return "buffer smaller than the plan";
    case KVC_E_BUDGET: return "workspace budget exceeded";
    case KVC_E_HIP: return "HIP runtime error";
    case KVC_E_NOMEM: return "host memory exhausted";
  }
  return "unknown status";
}

kvc_status kvc_plan(const kvc_layout* layout, const kvc_codec* codec, uint32_t n_pages, size_t* slot_bytes,
                    size_t* spill_bytes_suggested, size_t* bytes_per_token) {
  return no_throw([&]() -> kvc_status {
    kvc_status st = check_layout(layout);
    if (st == KVC_OK) st = check_codec(layout, codec);
    if (st != KVC_OK) return st;
    const Plan p = plan_totals(layout, codec, n_pages);
    const uint64_t raw_seg = align_up((uint64_t)layout->kv_heads * layout->tokens_per_page * layout->head_dim * 2,
                                      KVC_SLOT_ALIGN);
    if (slot_bytes) *slot_bytes = p.total;
    // ~3% of the fixed-size segments may fall back to raw, and every KVC_ANS16
    // segment needs its payload -- at most its raw size -- in the spill region
    if (spill_bytes_suggested)
      *spill_bytes_suggested = raw_seg * (std::max<uint64_t>(1, (p.encodable - p.ans + 31) / 32) + p.ans);
    if (bytes_per_token) *bytes_per_token = (p.per_page + layout->tokens_per_page - 1) / layout->tokens_per_page;
    return KVC_OK;
  });
}

kvc_status kvc_validate_encode(const kvc_layout* layout, const kvc_codec* codec, const int32_t* page_ids,
                               uint32_t n_pages, size_t out_bytes) {
  return no_throw([&]() -> kvc_status {
    kvc_status st = check_layout(layout);
    if (st == KVC_OK) st = check_codec(layout, codec);
    if (st == KVC_OK) st = check_grid(layout, n_pages);
    if (st == KVC_OK) st = check_pages(layout, page_ids, n_pages, false);
    if (st != KVC_OK) return st;
    if (plan_totals(layout, codec, n_pages).total > out_bytes) return KVC_E_CAPACITY;
    return KVC_OK;
  });
}

kvc_status kvc_validate_decode(const kvc_layout* layout, const kvc_codec* codec, const int32_t* dst_page_ids,
                               uint32_t n_pages, size_t in_bytes) {
  return no_throw([&]() -> kvc_status {
    kvc_status st = check_layout(layout);
    if (st == KVC_OK) st = check_codec(layout, codec);
    if (st == KVC_OK) st = check_grid(layout, n_pages);
    if (st == KVC_OK) st = check_pages(layout, dst_page_ids, n_pages, true);
    if (st != KVC_OK) return st;
    if (plan_totals(layout, codec, n_pages).total > in_bytes) return KVC_E_CAPACITY;
    return KVC_OK;
  });
}

kvc_status kvc_create(kvc_ctx** out, int hip_device, size_t workspace_budget) {
  return no_throw([&]() -> kvc_status {
    if (!out) return KVC_E_ARG;
    *out = nullptr;
    if (workspace_budget == 0) workspace_budget = KVC_DEFAULT_WORKSPACE;
    const size_t tb = tables_bytes() + cursor_pool_bytes();
    if (workspace_budget < tb + 4 * kAlign) return KVC_E_BUDGET;
    DeviceGuard g(hip_device);
    if (!g.ok) return KVC_E_HIP;
    // every host allocation that may throw comes before the device memory
    std::unique_ptr<Tables> t(new Tables());
    build_tables(*t);
    kvc_ctx* ctx = new kvc_ctx();
    ctx->device = hip_device;
    ctx->budget = workspace_budget;
    ctx->ring_begin = tb;
    ctx->ring_end = workspace_budget / kAlign * kAlign;
    ctx->head = ctx->ring_begin;
    bool ok = hipMalloc(&ctx->arena, workspace_budget) == hipSuccess &&
              hipHostMalloc(&ctx->staging, ctx->ring_end, hipHostMallocDefault) == hipSuccess &&
              hipMemcpy(ctx->arena, t.get(), sizeof(Tables), hipMemcpyHostToDevice) == hipSuccess &&
              hipMemset(ctx->arena + cursor_pool_offset(), 0, cursor_pool_bytes()) == hipSuccess &&
              hipDeviceSynchronize() == hipSuccess;
    if (!ok) {
      kvc_destroy(ctx);
      return KVC_E_HIP;
    }
    *out = ctx;
    return KVC_OK;
  });
}

kvc_status kvc_destroy(kvc_ctx* ctx) {
  return no_throw([&]() -> kvc_status {
    if (!ctx) return KVC_OK;
    kvc_status st = KVC_OK;
    {
      DeviceGuard g(ctx->device);
      for (auto& f : ctx->inflight) {
        if (hipEventSynchronize(f.ev) != hipSuccess) st = KVC_E_HIP;
        (void)hipEventDestroy(f.ev);
      }
      for (auto e : ctx->free_events) (void)hipEventDestroy(e);
      for (auto& ln : ctx->lane) {
        if (ln.last && hipEventSynchronize(ln.last) != hipSuccess) st = KVC_E_HIP;
        if (ln.ptr) (void)hipFree(ln.ptr);
        if (ln.last) (void)hipEventDestroy(ln.last);
      }
      reap_retired(ctx, true);
      if (ctx->copy_stream && hipStreamSynchronize(ctx->copy_stream) != hipSuccess) st = KVC_E_HIP;
      for (auto e : ctx->layer_copied) (void)hipEventDestroy(e);
      if (ctx->fork) (void)hipEventDestroy(ctx->fork);
      if (ctx->copy_stream) (void)hipStreamDestroy(ctx->copy_stream);
      if (ctx->arena) (void)hipFree(ctx->arena);
      if (ctx->staging) (void)hipHostFree(ctx->staging);
    }
    delete ctx;
    return st;
  });
}

kvc_status kvc_encode_pages(kvc_ctx* ctx, const kvc_layout* layout, const kvc_codec* codec,
                            const int32_t* page_ids, uint32_t n_pages, void* out, size_t out_bytes,
                            kvc_segment_desc* desc, void* stream) {
  return no_throw([&]() -> kvc_status {
    if (!ctx) return KVC_E_ARG;
    kvc_status st = kvc_validate_encode(layout, codec, page_ids, n_pages, out_bytes);
    if (st != KVC_OK) return st;
    if (n_pages == 0) return KVC_OK;
    if (!out || !desc || ((uintptr_t)out & 255) || ((uintptr_t)desc & 15)) return KVC_E_ARG;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVC_E_HIP;
    const HeapPlan plan(layout, codec, n_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    CallParams P{};
    size_t roff = 0, rsize = 0;
    st = stage_call(ctx, layout, codec, plan, page_ids, n_pages, s, &P, &roff, &rsize, true);
    if (st != KVC_OK) return st;
    P.buf = static_cast<uint8_t*>(out);
    P.buf_bytes = out_bytes;
    P.slot_region = plan.total;
    P.desc = desc;
    P.seg_status = nullptr;
    const uint64_t nseg = (uint64_t)layout->layers * n_pages * 2;
    if (run_encode(P, layout, plan, nseg, s) != hipSuccess) return KVC_E_HIP;
    return ring_commit(ctx, roff, rsize, s);
  });
}

kvc_status kvc_decode_pages(kvc_ctx* ctx, const kvc_layout* layout, const kvc_codec* codec, const void* in,
                            size_t in_bytes, const int32_t* dst_page_ids, uint32_t n_pages, uint8_t* seg_status,
                            void* stream) {
  return no_throw([&]() -> kvc_status {
    if (!ctx) return KVC_E_ARG;
    kvc_status st = kvc_validate_decode(layout, codec, dst_page_ids, n_pages, in_bytes);
    if (st != KVC_OK) return st;
    if (n_pages == 0) return KVC_OK;
    if (!in || ((uintptr_t)in & 255)) return KVC_E_ARG;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVC_E_HIP;
    const HeapPlan plan(layout, codec, n_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    CallParams P{};
    size_t roff = 0, rsize = 0;
    st = stage_call(ctx, layout, codec, plan, dst_page_ids, n_pages, s, &P, &roff, &rsize, false);
    if (st != KVC_OK) return st;
    P.buf = const_cast<uint8_t*>(static_cast<const uint8_t*>(in));
    P.buf_bytes = in_bytes;
    P.slot_region = plan.total;
    P.desc = nullptr;
    P.seg_status = seg_status;
    const uint64_t nseg = (uint64_t)layout->layers * n_pages * 2;
    if (run_decode(P, layout, plan, nseg, s) != hipSuccess) return KVC_E_HIP;
    return ring_commit(ctx, roff, rsize, s);
  });
}

kvc_status kvc_decode_layers(kvc_ctx* ctx, const kvc_layout* layout, const kvc_codec* codec, const void* in,
                             size_t in_bytes, const int32_t* dst_page_ids, uint32_t n_pages, uint32_t layer_begin,
                             uint32_t layer_end, uint8_t* seg_status, void* stream) {
  return no_throw([&]() -> kvc_status {
    if (!ctx) return KVC_E_ARG;
    kvc_status st = kvc_validate_decode(layout, codec, dst_page_ids, n_pages, in_bytes);
    if (st != KVC_OK) return st;
    if (layer_begin > layer_end || layer_end > layout->layers) return KVC_E_ARG;
    if (n_pages == 0 || layer_begin == layer_end) return KVC_OK;
    if (!in || ((uintptr_t)in & 255)) return KVC_E_ARG;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVC_E_HIP;
    const HeapPlan plan(layout, codec, n_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    CallParams P{};
    size_t roff = 0, rsize = 0;
    st = stage_call(ctx, layout, codec, plan, dst_page_ids, n_pages, s, &P, &roff, &rsize, false);
    if (st != KVC_OK) return st;
    P.buf = const_cast<uint8_t*>(static_cast<const uint8_t*>(in));
    P.buf_bytes = in_bytes;
    P.slot_region = plan.total;
    P.seg_status = seg_status;
    P.seg_base = layer_begin * n_pages * 2;
    if (run_decode(P, layout, plan, (uint64_t)(layer_end - layer_begin) * n_pages * 2, s) != hipSuccess)
      return KVC_E_HIP;
    return ring_commit(ctx, roff, rsize, s);
  });
}

kvc_status kvc_offload_pages(kvc_ctx* ctx, const kvc_layout* layout, const kvc_codec* codec_in,
                             const int32_t* page_ids, uint32_t n_pages, void* host_out, size_t host_bytes,
                             kvc_segment_desc* host_desc, size_t* host_used, void* stream) {
  return no_throw([&]() -> kvc_status {
    if (!ctx || !codec_in) return KVC_E_ARG;
    kvc_codec codec_crc = *codec_in;                 // the lane always stores a CRC32 per segment
    codec_crc.flags |= KVC_CODEC_CRC32;
    const kvc_codec* codec = &codec_crc;
    kvc_status st = kvc_validate_encode(layout, codec, page_ids, n_pages, host_bytes);
    if (st != KVC_OK) return st;
    if (host_used) *host_used = 0;
    if (n_pages == 0) return KVC_OK;
    const uint64_t nseg = (uint64_t)layout->layers * n_pages * 2;
    const size_t desc_bytes = nseg * sizeof(kvc_segment_desc);
    if (!pinned_range(host_out, host_bytes) || !pinned_range(host_desc, desc_bytes)) return KVC_E_ARG;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVC_E_HIP;
    const HeapPlan plan(layout, codec, n_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t buf_bytes = align_up(host_bytes, kAlign);
    st = lane_reserve(ctx, 0, buf_bytes + desc_bytes);
    if (st != KVC_OK) return st;
    auto& lane = ctx->lane[0];
    if (hipStreamWaitEvent(s, lane.last, 0) != hipSuccess) return KVC_E_HIP;   // the previous offload's copies
    CallParams P{};
    size_t roff = 0, rsize = 0;
    st = stage_call(ctx, layout, codec, plan, page_ids, n_pages, s, &P, &roff, &rsize, true);
    if (st != KVC_OK) return st;
    P.buf = lane.ptr;
    P.buf_bytes = host_bytes;
    P.slot_region = plan.total;
    P.desc = reinterpret_cast<kvc_segment_desc*>(lane.ptr + buf_bytes);
    if (run_encode(P, layout, plan, nseg, s) != hipSuccess) return KVC_E_HIP;
    // The spill bytes used are known only on the device: read the cursor
    // back once for the batch (into the host mirror of the call's own ring
    // bytes), start the slot and descriptor copies, then wait for the
    // encode and copy exactly the used spill bytes.
    unsigned long long* h_cursor = reinterpret_cast<unsigned long long*>(
        ctx->staging + (reinterpret_cast<uint8_t*>(P.spill_cursor) - ctx->arena));
    if (hipMemcpyAsync(h_cursor, P.spill_cursor, sizeof(*h_cursor), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipEventRecord(lane.last, s) != hipSuccess ||
        hipMemcpyAsync(host_out, lane.ptr, plan.total, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(host_desc, P.desc, desc_bytes, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipEventSynchronize(lane.last) != hipSuccess)
      return KVC_E_HIP;
    uint64_t cur = *h_cursor;
    if (P.cursor_lap)                            // a pool slot: this call's bytes, or none if another lap's tag
      cur = (cur >> kCursorLapShift) == P.cursor_lap ? cur & ((1ull << kCursorLapShift) - 1) : 0;
    const size_t used = std::min<size_t>((size_t)cur, host_bytes - plan.total);
    if ((used && hipMemcpyAsync(static_cast<uint8_t*>(host_out) + plan.total, lane.ptr + plan.total, used,
                                hipMemcpyDeviceToHost, s) != hipSuccess) ||
        hipEventRecord(lane.last, s) != hipSuccess)
      return KVC_E_HIP;
    if (host_used) *host_used = plan.total + used;
    return ring_commit(ctx, roff, rsize, s);
  });
}

kvc_status kvc_restore_pages(kvc_ctx* ctx, const kvc_layout* layout, const kvc_codec* codec_in, const void* host_in,
                             size_t in_bytes, const int32_t* dst_page_ids, uint32_t n_pages, uint32_t layer_begin,
                             uint32_t layer_end, uint8_t* seg_status, void* const* layer_ready, void* stream) {
  return no_throw([&]() -> kvc_status {
    if (!ctx || !codec_in) return KVC_E_ARG;
    kvc_codec codec_crc = *codec_in;                 // the lane always checks the segments' CRC32
    codec_crc.flags |= KVC_CODEC_CRC32;
    const kvc_codec* codec = &codec_crc;
    kvc_status st = kvc_validate_decode(layout, codec, dst_page_ids, n_pages, in_bytes);
    if (st != KVC_OK) return st;
    if (layer_begin > layer_end || layer_end > layout->layers) return KVC_E_ARG;
    if (n_pages == 0 || layer_begin == layer_end) return KVC_OK;
    if (!pinned_range(host_in, in_bytes)) return KVC_E_ARG;
    DeviceGuard g(ctx->device);
    if (!g.ok) return KVC_E_HIP;
    const HeapPlan plan(layout, codec, n_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t nl = layer_end - layer_begin;
    // lazily created: the copy stream (default priority), the fork event and
    // one copy-done event per layer of the widest restore so far
    if (!ctx->copy_stream && hipStreamCreateWithFlags(&ctx->copy_stream, hipStreamNonBlocking) != hipSuccess)
      return KVC_E_HIP;
    if (!ctx->fork && !(ctx->fork = new_event())) return KVC_E_HIP;
    ctx->layer_copied.reserve(nl);
    while (ctx->layer_copied.size() < nl) {
      hipEvent_t e = new_event();
      if (!e) return KVC_E_HIP;
      ctx->layer_copied.push_back(e);
    }
    st = lane_reserve(ctx, 1, align_up(in_bytes, kAlign));
    if (st != KVC_OK) return st;
    auto& lane = ctx->lane[1];
    CallParams P{};
    size_t roff = 0, rsize = 0;
    st = stage_call(ctx, layout, codec, plan, dst_page_ids, n_pages, s, &P, &roff, &rsize, false);
    if (st != KVC_OK) return st;
    P.buf = lane.ptr;
    P.buf_bytes = in_bytes;
    P.slot_region = plan.total;
    P.seg_status = seg_status;
    // The copy stream starts after the caller's earlier work (which may have
    // produced host_in) and after the previous restore's decodes have read the
    // staging buffer.
    const hipStream_t cs = ctx->copy_stream;
    const uint8_t* hin = static_cast<const uint8_t*>(host_in);
    if (hipEventRecord(ctx->fork, s) != hipSuccess || hipStreamWaitEvent(cs, ctx->fork, 0) != hipSuccess ||
        hipStreamWaitEvent(cs, lane.last, 0) != hipSuccess)
      return KVC_E_HIP;
    if (in_bytes > plan.total &&
        hipMemcpyAsync(lane.ptr + plan.total, hin + plan.total, in_bytes - plan.total, hipMemcpyHostToDevice, cs) !=
            hipSuccess)
      return KVC_E_HIP;
    for (uint32_t l = layer_begin; l < layer_end; l++) {
      const uint64_t a = plan.layer_off[l], b = l + 1 < layout->layers ? plan.layer_off[l + 1] : plan.total;
      hipEvent_t copied = ctx->layer_copied[l - layer_begin];
      if ((b > a && hipMemcpyAsync(lane.ptr + a, hin + a, b - a, hipMemcpyHostToDevice, cs) != hipSuccess) ||
          hipEventRecord(copied, cs) != hipSuccess || hipStreamWaitEvent(s, copied, 0) != hipSuccess)
        return KVC_E_HIP;
      P.seg_base = l * n_pages * 2;
      if (run_decode(P, layout, plan, (uint64_t)n_pages * 2, s) != hipSuccess) return KVC_E_HIP;
      if (layer_ready && layer_ready[l - layer_begin] &&
          hipEventRecord(static_cast<hipEvent_t>(layer_ready[l - layer_begin]), s) != hipSuccess)
        return KVC_E_HIP;
    }
    if (hipEventRecord(lane.last, s) != hipSuccess) return KVC_E_HIP;
    return ring_commit(ctx, roff, rsize, s);
  });
}

kvc_status kvc_encode_pages_noalloc(const kvc_layout* layout, const kvc_codec* codec, const int32_t* page_ids,
                                    uint32_t n_pages, void* out, size_t out_bytes, kvc_segment_desc* desc,
                                    void* stream) {
  return no_throw([&]() -> kvc_status {
    kvc_status st = check_layout(layout);
    if (st == KVC_OK) st = check_codec(layout, codec);
    if (st == KVC_OK) st = check_grid(layout, n_pages);
    if (st == KVC_OK) st = check_pages(layout, page_ids, n_pages, false);
    if (st != KVC_OK) return st;
    if (layout->layers > kNoAllocMaxLayers || n_pages > kNoAllocMaxPages) return KVC_E_BUDGET;
    // the plan in fixed arrays on the stack
    uint64_t layer_off[kNoAllocMaxLayers];
    uint32_t slot_k[kNoAllocMaxLayers], slot_v[kNoAllocMaxLayers];
    uint8_t eff_k[kNoAllocMaxLayers], eff_v[kNoAllocMaxLayers];
    Plan plan;
    plan.layer_off = layer_off;
    plan.slot[0] = slot_k;
    plan.slot[1] = slot_v;
    plan.eff[0] = eff_k;
    plan.eff[1] = eff_v;
    fill_plan(layout, codec, n_pages, plan);
    if (plan.total > out_bytes) return KVC_E_CAPACITY;
    if (n_pages == 0) return KVC_OK;
    if (!out || !desc || ((uintptr_t)out & 255) || ((uintptr_t)desc & 15)) return KVC_E_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KVC_E_HIP;
    uint8_t* scr = nullptr;
    if (noalloc_scratch(dev, static_tables(), &scr) != hipSuccess) return KVC_E_HIP;
    // host image of [spill cursor = 0 | side table], copied into the scratch
    // in one pageable copy (complete when the call returns)
    alignas(16) uint8_t img[kNoAllocSidesOff - kNoAllocCursorOff + sizeof(SideEntry) * 2 * kNoAllocMaxLayers];
    std::memset(img, 0, kNoAllocSidesOff - kNoAllocCursorOff);
    CallParams P{};
    fill_call(layout, codec, plan, n_pages, reinterpret_cast<SideEntry*>(img + (kNoAllocSidesOff - kNoAllocCursorOff)),
              &P);
    const size_t img_bytes = kNoAllocSidesOff - kNoAllocCursorOff + sizeof(SideEntry) * 2 * layout->layers;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(scr + kNoAllocCursorOff, img, img_bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipMemcpyAsync(scr + kNoAllocPagesOff, page_ids, sizeof(int32_t) * (size_t)n_pages, hipMemcpyHostToDevice,
                       s) != hipSuccess)
      return KVC_E_HIP;
    P.tables = reinterpret_cast<const Tables*>(scr);
    P.spill_cursor = reinterpret_cast<unsigned long long*>(scr + kNoAllocCursorOff);
    P.sides = reinterpret_cast<const SideEntry*>(scr + kNoAllocSidesOff);
    P.pages = reinterpret_cast<const int32_t*>(scr + kNoAllocPagesOff);
    P.buf = static_cast<uint8_t*>(out);
    P.buf_bytes = out_bytes;
    P.slot_region = plan.total;
    P.desc = desc;
    P.seg_status = nullptr;
    const uint64_t nseg = (uint64_t)layout->layers * n_pages * 2;
    return run_encode(P, layout, plan, nseg, s) == hipSuccess ? KVC_OK : KVC_E_HIP;
  });
}

}  // extern "C"
