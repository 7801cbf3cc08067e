// kvc_ans_device.h -- gfx950 kernels of the lossless entropy stage (KVC_ANS16),
// included by kvc_kernels.hip inside its namespace (they share its segment
// addressing, CRC and header helpers).
//
// OrbitKV docs, "KV precision and storage encoding", section "GPU ANS": typed
// 16-bit pages are entropy coded losslessly, decompression checks the exact
// output length, incompressible pages stay raw.  The coder is rANS (Duda,
// "Asymmetric numeral systems", 2013) over the low and high byte planes of a
// segment's values in canonical order, each plane with a static 12-bit model
// and 64 interleaved streams: element i belongs to stream (i / 8) mod 64.
// Payload layout (per plane, 16-byte aligned): u16 mode, u16 K, 12 zero
// bytes; mode 0: the n bytes; mode 1: a 32-byte presence bitmap, the K u16
// frequencies, 64 u16 stream lengths, the streams ([final state u32 LE]
// [renormalisation bytes, last emitted first]); zero padding to 16.
//
// One wave per segment: lane j owns stream j of both planes, i.e. the
// 8-element chunks c = j, j + 64, ... of the segment.

constexpr uint32_t kAnsStreams = 64;
constexpr uint32_t kAnsProbBits = 12;
constexpr uint32_t kAnsM = 1u << kAnsProbBits;
constexpr uint32_t kAnsL = 1u << 23;
constexpr int kAnsHistCopies = 4;              // sub-histograms: fewer lanes per LDS atomic address

// encode constants of one symbol: frequency, cumulative frequency and the
// reciprocal of the frequency for floor(x / f) = (x * m) >> (31 + l), exact
// for every x < 2^31 (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, Thm 4.2, with N = 31 and
// l = ceil(log2 f), m = ceil(2^(31+l) / f), which fits 32 bits for f <= 2^12)
struct AnsEnc {
  uint32_t f, cum, m, l;
};
struct AnsDec {
  uint16_t f, cum;
};

// element offset (in the page) of canonical chunk c: 8 elements of one vector
__device__ __forceinline__ uint32_t ans_chunk_off(const SegCtx& s, uint32_t c, uint32_t d) {
  const uint32_t i = 8 * c, v = i / d, e = i - v * d;
  const uint32_t t = (uint32_t)(((uint64_t)v * s.heads_magic) >> 32), h = v - t * (uint32_t)s.heads;
  return t * s.st + h * s.sh + e;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor(v, m, 64));
  return v;
}
// exclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= (uint32_t)o) x += y;
  }
  return x - v;
}

// the model of one plane from its 256 counts (symbols 4*lane .. 4*lane+3 in
// this lane): frequencies summing to 4096 -- each present symbol 1 plus its
// floored share of 4096 - K, the remainder to the most frequent (lowest on
// ties) -- and their cumulative sums; K is returned
__device__ __forceinline__ uint32_t ans_model(const uint32_t (&c)[4], uint32_t n, uint32_t (&f)[4],
                                              uint32_t (&cum)[4]) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t k = 0, key = 0;
  for (int r = 0; r < 4; r++) {
    k += c[r] != 0;
    key = max(key, (c[r] << 8) | (255u - (4 * lane + r)));          // count, then the lower symbol
  }
  k = wave_sum(k);
  key = wave_max(key);
  const uint32_t best = 255u - (key & 255u);
  uint32_t sum = 0;
  for (int r = 0; r < 4; r++) {
    f[r] = c[r] ? 1 + (c[r] * (kAnsM - k)) / n : 0;
    sum += f[r];
  }
  sum = wave_sum(sum);
  if (n && (best >> 2) == lane) f[best & 3] += kAnsM - sum;
  uint32_t run = wave_excl_scan(f[0] + f[1] + f[2] + f[3]);
  for (int r = 0; r < 4; r++) {
    cum[r] = run;
    run += f[r];
  }
  return k;
}

// one encode step: renormalise (at most two bytes), then x = C(s, x).
// EMIT: emitted byte k lands at end - 1 - k, for k below lim (the count of
// the sizing pass, so that a source changed between the passes cannot make
// the writes leave the stream's bytes)
template <bool EMIT>
__device__ __forceinline__ void ans_put(uint32_t& x, const AnsEnc& e, uint32_t& cnt, uint8_t* end, uint32_t lim) {
  const uint32_t x_max = (kAnsL >> kAnsProbBits << 8) * e.f;
#pragma unroll
  for (int r = 0; r < 2; r++)
    if (x >= x_max) {
      if constexpr (EMIT)
        if (cnt < lim) *(end - 1 - cnt) = (uint8_t)x;
      cnt++;
      x >>= 8;
    }
  const uint32_t q = (uint32_t)(((uint64_t)x * e.m) >> (31 + e.l));
  x = q * kAnsM + (x - q * e.f) + e.cum;
}

// encode both planes of lane j's stream in reverse element order; EMIT:
// write the renormalisation bytes before end0 / end1
template <int D, bool EMIT>
__device__ __forceinline__ void ans_encode_streams(const SegCtx& s, uint32_t n, const AnsEnc (*enc)[256],
                                                   const bool (&coded)[2], uint32_t (&x)[2], uint32_t (&cnt)[2],
                                                   uint8_t* end0, uint8_t* end1, uint32_t lim0, uint32_t lim1) {
  const uint32_t j = threadIdx.x & 63, chunks = n / 8;
  x[0] = x[1] = kAnsL;
  cnt[0] = cnt[1] = 0;
  if (j >= chunks) return;
  for (int c = (int)(j + (chunks - 1 - j) / kAnsStreams * kAnsStreams); c >= 0; c -= kAnsStreams) {
    const uint4 w = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, (uint32_t)c, D)));
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 7; e >= 0; e--) {
      const uint32_t v = (a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      if (coded[0]) ans_put<EMIT>(x[0], enc[0][v & 0xFF], cnt[0], end0, lim0);
      if (coded[1]) ans_put<EMIT>(x[1], enc[1][v >> 8], cnt[1], end1, lim1);
    }
  }
}

template <int D, bool CRC>
__global__ __launch_bounds__(64) void ans_encode_kernel(CallParams p) {
  __shared__ uint32_t s_hist[2][kAnsHistCopies][256];
  __shared__ AnsEnc s_enc[2][256];
  __shared__ unsigned long long s_off;
  CrcTables* const ct = crc_tables_lds<CRC>();
  const uint32_t seg = p.seg_base + blockIdx.x;
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry& E = p.sides[2 * l + comp];
  if (E.codec != C_ANS) return;
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = p.pages[pi];
  kvc_segment_desc* desc = p.desc + seg;
  const uint32_t lane = threadIdx.x;
  if ((uint64_t)(uintptr_t)E.base < p.base_lo || (uint64_t)(uintptr_t)E.base > p.base_hi || page < 0 ||
      (uint32_t)page >= p.num_blocks || slot_off + E.slot_bytes > p.slot_region) {
    if (lane == 0) reinterpret_cast<uint4*>(desc)[1] = make_uint4(0, 0, (uint32_t)KVC_SEG_GUARD << 24, 0);
    return;
  }
  SegCtx s;
  s.src = E.base + (int64_t)page * p.sb;
  s.slot = p.buf + slot_off;
  s.heads = (int)p.heads;
  s.heads_magic = p.heads_magic;
  s.n_vec = (int)(p.heads * p.tokens);
  s.st = p.st32;
  s.sh = p.sh32;
  const uint32_t n = (uint32_t)s.n_vec * D, raw_bytes = 2 * n, chunks = n / 8;
  constexpr int crc_flag = CRC ? KVC_FLAG_CRC32 : 0;
  if constexpr (CRC) load_crc_tables<64>(ct, &p.tables->crc);

  // histograms of both planes
  for (uint32_t u = lane; u < 2 * kAnsHistCopies * 256; u += 64) (&s_hist[0][0][0])[u] = 0;
  __syncthreads();
  for (uint32_t c = lane; c < chunks; c += kAnsStreams) {
    const uint4 w = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, c, D)));
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t v = (a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      atomicAdd(&s_hist[0][lane & (kAnsHistCopies - 1)][v & 0xFF], 1u);
      atomicAdd(&s_hist[1][lane & (kAnsHistCopies - 1)][v >> 8], 1u);
    }
  }
  __syncthreads();
  // models, encode constants, and pass 1: the stream lengths
  uint32_t f[2][4], cum[2][4], k[2];
  for (int pl = 0; pl < 2; pl++) {
    uint32_t c[4];
    for (int r = 0; r < 4; r++) {
      c[r] = 0;
      for (int q = 0; q < kAnsHistCopies; q++) c[r] += s_hist[pl][q][4 * lane + r];
    }
    k[pl] = ans_model(c, n, f[pl], cum[pl]);
    for (int r = 0; r < 4; r++) {
      const uint32_t d = f[pl][r], lg = d > 1 ? 32 - __clz(d - 1) : 0;
      const uint32_t m = d ? (uint32_t)((((uint64_t)1 << (31 + lg)) + d - 1) / d) : 0;
      s_enc[pl][4 * lane + r] = AnsEnc{d, cum[pl][r], m, lg};
    }
  }
  __syncthreads();
  const bool all[2] = {true, true};
  uint32_t x[2], cnt[2];
  ans_encode_streams<D, false>(s, n, s_enc, all, x, cnt, nullptr, nullptr, 0, 0);
  uint32_t len[2], body[2], psize[2];
  bool coded[2];
  for (int pl = 0; pl < 2; pl++) {
    len[pl] = 4 + cnt[pl];
    body[pl] = 32 + 2 * k[pl] + 2 * kAnsStreams + wave_sum(len[pl]);
    coded[pl] = body[pl] < n;
    psize[pl] = (16 + (coded[pl] ? body[pl] : n) + 15) & ~15u;
  }
  const uint32_t payload = psize[0] + psize[1];
  const bool keep = 8 * (E.slot_bytes + ((payload + 255) & ~255u)) <= 7 * raw_bytes;
  const uint32_t need = keep ? ((payload + 255) & ~255u) : ((raw_bytes + 255) & ~255u);
  if (lane == 0) s_off = atomicAdd(p.spill_cursor, (unsigned long long)need);
  __syncthreads();
  const uint64_t off = p.slot_region + s_off;
  const bool fits = off + need <= p.buf_bytes;
  uint8_t* const heap = p.buf + off;
  // the slot: header (written last) and zeros
  for (uint32_t u = 2 + lane; u < E.slot_bytes / 16; u += 64) st_global16(s.slot + 16 * u, make_uint4(0, 0, 0, 0));
  if (!fits) {                                                   // no room: not stored
    if (lane == 0)
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_DATA | KVC_FLAG_CAPACITY, KVC_SEG_CAPACITY,
                        (int)p.dtype, comp, D, s.n_vec, raw_bytes, 0, 0, 0);
    return;
  }
  if (!keep) {                                                   // incompressible: raw bytes in the spill
    for (uint32_t c = lane; c < chunks; c += kAnsStreams)
      st_global16(heap + 16 * c, ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, c, D))));
    const uint32_t cr = CRC ? crc32_written(heap, raw_bytes, ct) : 0u;
    if (lane == 0)
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_DATA | crc_flag, KVC_SEG_RAW_DATA,
                        (int)p.dtype, comp, D, s.n_vec, raw_bytes, off, 0, cr);
    return;
  }
  // pass 2: the payload
  uint32_t base[2] = {0, psize[0]};
  uint8_t* end[2] = {nullptr, nullptr};
  for (int pl = 0; pl < 2; pl++) {
    uint8_t* const P = heap + base[pl];
    if (lane == 0) {
      st_global16(P, make_uint4(coded[pl] ? 1u | (k[pl] << 16) : 0u, 0, 0, 0));
      for (uint32_t b = 16 + (coded[pl] ? body[pl] : n); b < psize[pl]; b++) P[b] = 0;
    }
    if (!coded[pl]) {                                            // raw plane: byte pl of every value
      for (uint32_t c = lane; c < chunks; c += kAnsStreams) {
        const uint4 w = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, c, D)));
        const uint32_t sel = pl ? 0x07050301u : 0x06040200u;    // bytes of the 8 values, in order
        *reinterpret_cast<uint2*>(P + 16 + 8 * c) =
            make_uint2(__builtin_amdgcn_perm(w.y, w.x, sel), __builtin_amdgcn_perm(w.w, w.z, sel));
      }
      continue;
    }
    // bitmap, frequencies of the present symbols, stream lengths
    uint32_t nib = 0, present = 0;
    for (int r = 0; r < 4; r++) {
      nib |= (f[pl][r] != 0) << r;
      present += f[pl][r] != 0;
    }
    const uint32_t other = __shfl_xor(nib, 1, 64);
    if (!(lane & 1)) P[16 + lane / 2] = (uint8_t)(nib | (other << 4));
    uint32_t pos = wave_excl_scan(present);
    for (int r = 0; r < 4; r++)
      if (f[pl][r]) *reinterpret_cast<uint16_t*>(P + 48 + 2 * pos++) = (uint16_t)f[pl][r];
    uint8_t* const lens = P + 48 + 2 * k[pl];
    *reinterpret_cast<uint16_t*>(lens + 2 * lane) = (uint16_t)len[pl];
    uint8_t* const st = lens + 2 * kAnsStreams + wave_excl_scan(len[pl]);
    end[pl] = st + len[pl];
  }
  ans_encode_streams<D, true>(s, n, s_enc, coded, x, cnt, end[0], end[1], len[0] - 4, len[1] - 4);
  for (int pl = 0; pl < 2; pl++)
    if (coded[pl]) {
      uint8_t* const st = end[pl] - len[pl];
      st[0] = (uint8_t)x[pl];
      st[1] = (uint8_t)(x[pl] >> 8);
      st[2] = (uint8_t)(x[pl] >> 16);
      st[3] = (uint8_t)(x[pl] >> 24);
    }
  const uint32_t cr = CRC ? crc32_written(heap, payload, ct) : 0u;
  if (lane == 0) {
    __threadfence();                                             // payload before the header that points at it
    write_header_desc(s.slot, desc, slot_off, C_ANS, KVC_FLAG_HEAP | crc_flag, KVC_SEG_ENCODED, (int)p.dtype,
                      comp, D, s.n_vec, payload, off, 0, cr);
  }
}

// slot -> symbol table of a coded plane and its (f, cum) pairs; returns
// false if the plane's model is malformed.  Lanes fill 64-slot blocks.
__device__ __forceinline__ bool ans_load_model(const uint8_t* P, uint32_t k, AnsDec* tab, uint8_t* lut) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t fr[4], present = 0;
  for (int r = 0; r < 4; r++) present += (P[16 + (4 * lane + r) / 8] >> ((4 * lane + r) & 7)) & 1;
  uint32_t pos = wave_excl_scan(present);
  const bool ok_k = wave_sum(present) == k;
  uint32_t tot = 0;
  for (int r = 0; r < 4; r++) {
    const uint32_t sy = 4 * lane + r;
    fr[r] = ((P[16 + sy / 8] >> (sy & 7)) & 1) && pos < k ? *reinterpret_cast<const uint16_t*>(P + 48 + 2 * pos++) : 0;
    tot += fr[r];
  }
  bool ok = ok_k && wave_sum(tot) == kAnsM;
  for (int r = 0; r < 4; r++) ok = ok && (((P[16 + (4 * lane + r) / 8] >> ((4 * lane + r) & 7)) & 1) == (fr[r] != 0));
  ok = __all(ok);
  uint32_t run = wave_excl_scan(tot);
  for (int r = 0; r < 4; r++) {
    tab[4 * lane + r] = AnsDec{(uint16_t)fr[r], (uint16_t)run};
    run += fr[r];
  }
  __syncthreads();
  if (!ok) return false;
  // slots [64*lane, 64*lane + 64): the symbol of the first by binary search, then walk
  const uint32_t s0 = 64 * lane;
  uint32_t lo = 0, hi = 255;                                     // largest symbol with cum <= s0 and f > 0
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (tab[mid].cum <= s0) lo = mid;
    else hi = mid - 1;
  }
  uint32_t sy = lo;
  while (sy > 0 && tab[sy].f == 0) sy--;
  for (uint32_t sl = s0; sl < s0 + 64; sl++) {
    while (sl >= (uint32_t)tab[sy].cum + tab[sy].f) sy++;
    lut[sl] = (uint8_t)sy;
  }
  __syncthreads();
  return true;
}

template <int D, bool CRC>
__global__ __launch_bounds__(64) void ans_decode_kernel(CallParams p) {
  __shared__ AnsDec s_tab[2][256];
  __shared__ uint8_t s_lut[2][kAnsM];
  __shared__ uint32_t s_crc_ok;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_img[];  // p.stage_bytes: the payload
  CrcTables* const ct = crc_tables_lds<CRC>();
  const uint32_t seg = p.seg_base + blockIdx.x;
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry& E = p.sides[2 * l + comp];
  if (E.codec != C_ANS) return;
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = p.pages[pi];
  const uint32_t lane = threadIdx.x;
  const bool report = p.seg_status && lane == 0;
  if ((uint64_t)(uintptr_t)E.base < p.base_lo || (uint64_t)(uintptr_t)E.base > p.base_hi || page < 0 ||
      (uint32_t)page >= p.num_blocks || slot_off + E.slot_bytes > p.slot_region) {
    if (report) p.seg_status[seg] = 2;
    return;
  }
  SegCtx s;
  s.src = E.base + (int64_t)page * p.sb;                         // destination page
  s.slot = p.buf + slot_off;
  s.heads = (int)p.heads;
  s.heads_magic = p.heads_magic;
  s.n_vec = (int)(p.heads * p.tokens);
  s.st = p.st32;
  s.sh = p.sh32;
  uint16_t* const page_p = const_cast<uint16_t*>(s.src);
  const uint32_t n = (uint32_t)s.n_vec * D, raw_bytes = 2 * n, chunks = n / 8;
  if constexpr (CRC) load_crc_tables<64>(ct, &p.tables->crc);
  const uint4 h0 = ld_global16(s.slot), h1 = ld_global16(s.slot + 16);
  const int version = h0.x & 0xFF, format = (h0.x >> 8) & 0xFF, flags = (h0.x >> 16) & 0xFF;
  const int dc = (h0.x >> 24) & 0xFF;
  bool ok = version == 1 && dc == ((int)p.dtype | (int)(comp << 4)) && (h0.y & 0xFFFF) == (uint32_t)D &&
            (h0.y >> 16) == (uint32_t)s.n_vec && h0.z == raw_bytes && ((flags & KVC_FLAG_CRC32) != 0) == CRC;
  const bool raw_data = flags & KVC_FLAG_RAW_DATA;
  const uint64_t spill = (uint64_t)h1.x | ((uint64_t)h1.y << 32);
  const uint32_t stored = h0.w;
  if (raw_data) ok = ok && format == KVC_RAW && !(flags & KVC_FLAG_CAPACITY) && stored == raw_bytes;
  else ok = ok && format == C_ANS && (flags & KVC_FLAG_HEAP) && stored >= 32 && stored <= p.stage_bytes;
  // every read stays in the buffer: the stored bytes rounded up to 16
  const uint64_t span = ((uint64_t)stored + 15) & ~15ull;
  ok = ok && spill >= p.slot_region && span <= p.buf_bytes && spill <= p.buf_bytes - span;
  if (!ok) {
    if (report) p.seg_status[seg] = 1;
    return;
  }
  const uint8_t* const heap = p.buf + spill;
  if constexpr (CRC) {
    __syncthreads();
    const uint32_t c = crc32_wave(GlobalBytes{heap}, stored, ct);
    if (lane == 0) s_crc_ok = c == h1.z;
    __syncthreads();
    if (!s_crc_ok) {
      if (report) p.seg_status[seg] = 3;
      return;
    }
  }
  if (raw_data) {
    for (uint32_t c = lane; c < chunks; c += kAnsStreams)
      st_global16(byte_at(page_p, 2 * ans_chunk_off(s, c, D)), ld_global16(heap + 16 * c));
    if (report) p.seg_status[seg] = 0;
    return;
  }
  // stage the payload, parse both planes' headers and models
  for (uint32_t u = lane; u < (stored + 15) / 16; u += 64)
    *reinterpret_cast<uint4*>(s_img + 16 * u) = ld_global16(heap + 16 * u);
  __syncthreads();
  uint32_t pbase[2], mode[2], kk[2], sbeg[2] = {0, 0}, send[2] = {0, 0};
  uint32_t at = 0;
  bool good = true;
  for (int pl = 0; pl < 2 && good; pl++) {
    const uint8_t* const P = s_img + at;
    pbase[pl] = at;
    good = at + 16 <= stored;
    if (!good) break;
    const uint4 hd = *reinterpret_cast<const uint4*>(P);
    mode[pl] = hd.x & 0xFFFF;
    kk[pl] = hd.x >> 16;
    good = hd.y == 0 && hd.z == 0 && hd.w == 0 && mode[pl] <= 1 && kk[pl] <= 256;
    if (!good) break;
    uint32_t size;
    if (mode[pl] == 0) {
      good = kk[pl] == 0;
      size = 16 + n;
    } else {
      const uint32_t lens_at = at + 48 + 2 * kk[pl];
      good = lens_at + 2 * kAnsStreams <= stored && kk[pl] >= 1;
      if (!good) break;
      const uint32_t len = *reinterpret_cast<const uint16_t*>(s_img + lens_at + 2 * lane);
      const uint32_t st0 = lens_at + 2 * kAnsStreams + wave_excl_scan(len);
      sbeg[pl] = st0;
      send[pl] = st0 + len;
      good = __all(len >= 4) && wave_max(st0 + len) <= stored;
      size = 48 + 2 * kk[pl] + 2 * kAnsStreams + wave_sum(len);
      if (good) good = ans_load_model(P, kk[pl], s_tab[pl], s_lut[pl]);
    }
    const uint32_t padded = (size + 15) & ~15u;
    good = good && at + padded <= stored;
    if (good) good = __all(lane >= padded - size || s_img[at + size + lane] == 0);   // zero padding
    at += padded;
  }
  good = good && at == stored;                                   // exact length of the payload
  if (!good) {
    if (report) p.seg_status[seg] = 1;
    return;
  }
  // decode lane j's streams of both planes, writing each chunk of 8 values
  uint32_t x[2] = {kAnsL, kAnsL}, pos[2] = {sbeg[0], sbeg[1]};
  for (int pl = 0; pl < 2; pl++)
    if (mode[pl]) {                                              // final state, u32 little-endian
      const uint8_t* q = s_img + pos[pl];
      x[pl] = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
      pos[pl] += 4;
    }
  bool bad = false;
  for (uint32_t c = lane; c < chunks; c += kAnsStreams) {
    uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t i = 8 * c + e;
      uint32_t b[2];
#pragma unroll
      for (int pl = 0; pl < 2; pl++) {
        if (!mode[pl]) {
          b[pl] = s_img[pbase[pl] + 16 + i];
          continue;
        }
        const uint32_t sl = x[pl] & (kAnsM - 1), sy = s_lut[pl][sl];
        const AnsDec t = s_tab[pl][sy];
        b[pl] = sy;
        x[pl] = t.f * (x[pl] >> kAnsProbBits) + sl - t.cum;
#pragma unroll
        for (int r = 0; r < 2; r++)
          if (x[pl] < kAnsL) {
            const bool in = pos[pl] < send[pl];
            bad |= !in;
            x[pl] = (x[pl] << 8) | (in ? s_img[pos[pl]] : 0u);
            pos[pl] += in;
          }
      }
      o[e >> 1] |= (b[0] | (b[1] << 8)) << (16 * (e & 1));
    }
    st_global16(byte_at(page_p, 2 * ans_chunk_off(s, c, D)), make_uint4(o[0], o[1], o[2], o[3]));
  }
  for (int pl = 0; pl < 2; pl++) bad |= mode[pl] && (pos[pl] != send[pl] || x[pl] != kAnsL);
  bad = __any(bad);
  if (report) p.seg_status[seg] = bad ? 1 : 0;
}

template <int D, bool CRC>
void launch_ans_encode_dc(const CallParams& p, uint64_t n, hipStream_t st) {
  hipLaunchKernelGGL((ans_encode_kernel<D, CRC>), dim3((unsigned)n), dim3(64), 0, st, p);
}
template <int D, bool CRC>
void launch_ans_decode_dc(const CallParams& p, uint64_t n, hipStream_t st) {
  hipLaunchKernelGGL((ans_decode_kernel<D, CRC>), dim3((unsigned)n), dim3(64), p.stage_bytes, st, p);
}
