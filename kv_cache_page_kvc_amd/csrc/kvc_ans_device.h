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

// encode constants of one symbol with frequency f and cumulative frequency
// cum, for the state update x -> (x / f) * 4096 + x mod f + cum written as
// x + bias + q * cmpl with q = floor(x / f), cmpl = 4096 - f, bias = cum.
// q is the high word of x * rcp shifted right by shift: rcp = ceil(2^(31+l)
// / f), shift = l - 1 with l = ceil(log2 f), exact for every x < 2^31
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, Thm 4.2, with N = 31).  For f = 1, rcp =
// 2^32 - 1 and shift = 0 give q = x - 1, and bias = cum + 4095 restores
// x * 4096 + cum.  x_max = f * 2^19 bounds the state before the update.
struct AnsEnc {
  uint32_t x_max, rcp, bias, cmpl_shift;       // cmpl | shift << 16
};
struct AnsDec {
  uint16_t f, cum;
};
__device__ __forceinline__ AnsEnc ans_enc_entry(uint32_t f, uint32_t cum, const uint32_t* rcp_tab) {
  if (f == 0) return AnsEnc{0, 0, 0, 0};
  if (f == 1) return AnsEnc{1u << 19, 0xFFFFFFFFu, cum + kAnsM - 1, kAnsM - 1};
  const uint32_t l = 32 - __clz(f - 1);
  return AnsEnc{f << 19, rcp_tab[f], cum, (kAnsM - f) | ((l - 1) << 16)};
}

// LDS of the encode kernel (dynamic): the histograms -- the high byte plane
// in kAnsHiCopies copies, the low in kAnsLoCopies, copy-minor so that lanes
// counting one symbol in different copies hit different banks -- then, in
// the same bytes, the encode constants of both planes followed by the image
// of one coded plane (p.stage_bytes: its 16-byte header, model, lengths and
// streams, at most n + 16 bytes).
constexpr uint32_t kAnsHiCopies = 16, kAnsLoCopies = 4;
constexpr uint32_t kAnsHistAhead = 8;                    // histogram pass: source chunks in flight per lane
constexpr uint32_t kAnsHistBytes = 4 * 256 * (kAnsHiCopies + kAnsLoCopies);
constexpr uint32_t kAnsEncBytes = 2 * 256 * sizeof(AnsEnc);
inline uint32_t ans_encode_lds(uint32_t stage_bytes) {
  return kAnsHistBytes > kAnsEncBytes + stage_bytes ? kAnsHistBytes : kAnsEncBytes + stage_bytes;
}

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

// one encode step: renormalise, then x = C(s, x).  The state leaves k bytes,
// low byte first: one when x >= x_max, a second when also x >= 256 x_max
// (never a third: x < 2^31 and x_max >= 2^19).  EMIT: emitted byte number
// cnt lands at out[end - 1 - cnt] for cnt below lim (the count of the sizing
// pass, so that a source changed between the passes cannot make the writes
// leave the stream's bytes).  q = floor(x / f) < 2^19 and cmpl < 2^12, so
// their product is a 24-bit multiply.
template <bool EMIT>
__device__ __forceinline__ void ans_put(uint32_t& x, const AnsEnc& e, uint32_t& cnt, uint8_t* out, uint32_t end,
                                        uint32_t lim) {
  const bool one = x >= e.x_max, two = e.x_max < (1u << 24) && x >= (e.x_max << 8);
  if constexpr (EMIT) {
    if (one && cnt < lim) out[end - 1 - cnt] = (uint8_t)x;
    if (two && cnt + 1 < lim) out[end - 2 - cnt] = (uint8_t)(x >> 8);
  }
  const uint32_t k = (uint32_t)one + (uint32_t)two;
  cnt += k;
  x >>= 8 * k;
  const uint32_t q = __umulhi(x, e.rcp) >> (e.cmpl_shift >> 16);
  x = x + e.bias + __umul24(q, e.cmpl_shift & 0xFFFFu);
}

// encode the planes in use (U0: low, U1: high) of lane j's stream in reverse
// element order; EMIT: write the renormalisation bytes of plane pl before
// out[end[pl]].  RAW = 0 / 1: also store byte plane RAW of each chunk, in
// order, at raw[8 c] (the raw plane of the payload).  The next chunk's
// source is loaded while this one is coded, and a chunk's encode constants
// are read before its first step.
template <int D, bool EMIT, bool U0, bool U1, int RAW = -1>
__device__ __forceinline__ void ans_encode_streams(const SegCtx& s, uint32_t n, const AnsEnc* enc,
                                                   uint32_t (&x)[2], uint32_t (&cnt)[2], uint8_t* out,
                                                   const uint32_t (&end)[2], const uint32_t (&lim)[2],
                                                   uint8_t* raw = nullptr) {
  const uint32_t j = threadIdx.x & 63, chunks = n / 8;
  x[0] = x[1] = kAnsL;
  cnt[0] = cnt[1] = 0;
  if (j >= chunks) return;
  int c = (int)(j + (chunks - 1 - j) / kAnsStreams * kAnsStreams);
  uint4 nw = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, (uint32_t)c, D)));
  for (; c >= 0; c -= kAnsStreams) {
    const uint32_t a[4] = {nw.x, nw.y, nw.z, nw.w};
    if (c >= (int)kAnsStreams) nw = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, (uint32_t)c - kAnsStreams, D)));
    if constexpr (RAW >= 0) {
      constexpr uint32_t sel = RAW ? 0x07050301u : 0x06040200u;  // byte RAW of the 8 values, in order
      st_global8(raw + 8 * c, make_uint2(__builtin_amdgcn_perm(a[1], a[0], sel), __builtin_amdgcn_perm(a[3], a[2], sel)));
    }
    AnsEnc e0[8], e1[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t v = (a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      if constexpr (U0) e0[e] = enc[v & 0xFF];
      if constexpr (U1) e1[e] = enc[256 + (v >> 8)];
    }
#pragma unroll
    for (int e = 7; e >= 0; e--) {
      if constexpr (U0) ans_put<EMIT>(x[0], e0[e], cnt[0], out, end[0], lim[0]);
      if constexpr (U1) ans_put<EMIT>(x[1], e1[e], cnt[1], out, end[1], lim[1]);
    }
  }
}

// True when a plane's coded body (32-byte bitmap, 2K bytes of frequencies,
// 128 of stream lengths, the 64 streams: 4 state bytes each plus B_j
// renormalisation bytes) cannot be below n bytes, so the plane is stored raw
// without a sizing pass.  A coding step from a state x in [2^23, 2^31) that
// emits b bytes gives a state above x 2^(-8b) (4096 / f) (1 - 2^-11)^2
// (floor(x / f) > x / f - 1 with x 2^(-8b) >= 2^11 f, and the same for the
// shift), so over a stream from 2^23 to a final state below 2^31,
// 8 B_j > (bits of its symbols) - 8 - 0.00141 m_j, and over the plane
// 8 sum B_j > H - 512 - 0.00141 n with H = sum of count(s) log2(4096 / f(s)).
// H is evaluated in binary32 to well within the 2^-10 relative margin taken.
__device__ __forceinline__ bool ans_raw_certain(const uint32_t (&c)[4], const uint32_t (&f)[4], uint32_t k,
                                                uint32_t n) {
  float h = 0.0f;
  for (int r = 0; r < 4; r++)
    if (f[r]) h += (float)c[r] * (12.0f - log2f((float)f[r]));
  for (int m = 32; m >= 1; m >>= 1) h += __shfl_xor(h, m, 64);
  const float bits = h * (1.0f - 1.0f / 1024.0f) - 512.0f - 0.002f * (float)n;
  return 416.0f + 2.0f * (float)k + bits / 8.0f >= (float)n + 1.0f;
}

template <int D, bool CRC>
__global__ __launch_bounds__(64) void ans_encode_kernel(CallParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  uint32_t* const s_hist_hi = reinterpret_cast<uint32_t*>(s_dyn);     // [256][kAnsHiCopies]
  uint32_t* const s_hist_lo = s_hist_hi + 256 * kAnsHiCopies;         // [256][kAnsLoCopies]
  AnsEnc* const s_enc = reinterpret_cast<AnsEnc*>(s_dyn);             // [2][256], after the histograms
  uint8_t* const s_out = s_dyn + kAnsEncBytes;                        // one coded plane's image
  __shared__ unsigned long long s_off;
  CrcLds* const ct = crc_tables_lds<CRC>();
  const uint32_t seg = p.seg_base + blockIdx.x;
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry E = side_entry(p, 2 * l + comp);
  if (E.codec != C_ANS) return;
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = page_id(p, pi);
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
  if (n + 16 > p.stage_bytes) {                                  // the launch's LDS cannot hold a plane image
    if (lane == 0) reinterpret_cast<uint4*>(desc)[1] = make_uint4(0, 0, (uint32_t)KVC_SEG_GUARD << 24, 0);
    return;
  }
  constexpr int crc_flag = CRC ? KVC_FLAG_CRC32 : 0;
  if constexpr (CRC) load_crc_tables<64>(ct, &p.tables->crc);

  // histograms of both planes
  for (uint32_t u = lane; u < kAnsHistBytes / 16; u += 64) reinterpret_cast<uint4*>(s_dyn)[u] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  // kAnsHistAhead chunks per lane in flight: with one wave per segment and
  // few waves per CU, a single outstanding load per lane leaves this phase
  // bound by load latency
  uint4 nw[kAnsHistAhead];
#pragma unroll
  for (uint32_t q = 0; q < kAnsHistAhead; q++) {
    const uint32_t c = lane + q * kAnsStreams;
    nw[q] = c < chunks ? ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, c, D))) : make_uint4(0, 0, 0, 0);
  }
  for (uint32_t c0 = lane; c0 < chunks; c0 += kAnsHistAhead * kAnsStreams) {
#pragma unroll
    for (uint32_t q = 0; q < kAnsHistAhead; q++) {
      const uint32_t c = c0 + q * kAnsStreams, cn = c + kAnsHistAhead * kAnsStreams;
      if (c >= chunks) break;
      const uint32_t a[4] = {nw[q].x, nw[q].y, nw[q].z, nw[q].w};
      if (cn < chunks) nw[q] = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, cn, D)));
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const uint32_t v = (a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        atomicAdd(&s_hist_lo[(v & 0xFF) * kAnsLoCopies + (lane & (kAnsLoCopies - 1))], 1u);
        atomicAdd(&s_hist_hi[(v >> 8) * kAnsHiCopies + (lane & (kAnsHiCopies - 1))], 1u);
      }
    }
  }
  __syncthreads();
  // counts of symbols 4*lane .. 4*lane+3, then the models and encode constants
  uint32_t cnts[2][4];
  for (int r = 0; r < 4; r++) {
    const uint32_t sy = 4 * lane + r;
    uint32_t t = 0;
    for (uint32_t q = 0; q < kAnsLoCopies; q++) t += s_hist_lo[sy * kAnsLoCopies + q];
    cnts[0][r] = t;
    t = 0;
    for (uint32_t q = 0; q < kAnsHiCopies; q++) t += s_hist_hi[sy * kAnsHiCopies + q];
    cnts[1][r] = t;
  }
  __syncthreads();                                               // the constants overwrite the histograms
  uint32_t f[2][4], cum[2][4], k[2];
  for (int pl = 0; pl < 2; pl++) {
    k[pl] = ans_model(cnts[pl], n, f[pl], cum[pl]);
    for (int r = 0; r < 4; r++) s_enc[256 * pl + 4 * lane + r] = ans_enc_entry(f[pl][r], cum[pl][r], p.tables->ans_rcp);
  }
  __syncthreads();
  // pass 1: the stream lengths of the planes that may code below raw size
  const bool sure_raw[2] = {ans_raw_certain(cnts[0], f[0], k[0], n), ans_raw_certain(cnts[1], f[1], k[1], n)};
  const uint32_t zero2[2] = {0, 0};
  uint32_t x[2] = {kAnsL, kAnsL}, cnt[2] = {0, 0};
  if (!sure_raw[0] && !sure_raw[1]) ans_encode_streams<D, false, true, true>(s, n, s_enc, x, cnt, nullptr, zero2, zero2);
  else if (!sure_raw[0]) ans_encode_streams<D, false, true, false>(s, n, s_enc, x, cnt, nullptr, zero2, zero2);
  else if (!sure_raw[1]) ans_encode_streams<D, false, false, true>(s, n, s_enc, x, cnt, nullptr, zero2, zero2);
  uint32_t len[2], body[2], psize[2];
  bool coded[2];
  for (int pl = 0; pl < 2; pl++) {
    len[pl] = 4 + cnt[pl];
    body[pl] = 32 + 2 * k[pl] + 2 * kAnsStreams + wave_sum(len[pl]);
    coded[pl] = !sure_raw[pl] && body[pl] < n;
    psize[pl] = (16 + (coded[pl] ? body[pl] : n) + 15) & ~15u;
  }
  const uint32_t payload = psize[0] + psize[1];
  const bool keep = 8 * (E.slot_bytes + ((payload + 255) & ~255u)) <= 7 * raw_bytes;
  const uint32_t need = keep ? ((payload + 255) & ~255u) : ((raw_bytes + 255) & ~255u);
  if (lane == 0) s_off = spill_reserve(p, need);
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
    for (uint32_t c0 = lane; c0 < chunks; c0 += 4 * kAnsStreams) {
      uint4 w[4];
#pragma unroll
      for (uint32_t u = 0; u < 4; u++)
        if (c0 + u * kAnsStreams < chunks) w[u] = ld_global16(byte_at(s.src, 2 * ans_chunk_off(s, c0 + u * kAnsStreams, D)));
#pragma unroll
      for (uint32_t u = 0; u < 4; u++)
        if (c0 + u * kAnsStreams < chunks) st_global16(heap + 16 * (c0 + u * kAnsStreams), w[u]);
    }
    const uint32_t cr = CRC ? crc32_written<64>(heap, raw_bytes, ct, p.tables) : 0u;
    if (lane == 0)
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_DATA | crc_flag, KVC_SEG_RAW_DATA,
                        (int)p.dtype, comp, D, s.n_vec, raw_bytes, off, 0, cr);
    return;
  }
  // pass 2, a coded plane at a time, assembled in LDS and written out in
  // 16-byte units; a raw plane (at most one: two raw planes fail the keep
  // rule) is written during the coded plane's pass.  16 + n is a multiple of
  // 16, so a raw plane has no padding.
  uint8_t* const P0 = heap;
  uint8_t* const P1 = heap + psize[0];
  const int rawpl = coded[0] ? (coded[1] ? -1 : 1) : 0;
  if (rawpl >= 0 && lane == 0) st_global16(rawpl ? P1 : P0, make_uint4(0, 0, 0, 0));   // mode 0, K = 0
#pragma unroll
  for (int pl = 0; pl < 2; pl++) {
    uint8_t* const P = pl ? P1 : P0;
    if (!coded[pl]) continue;
    // header, bitmap, frequencies of the present symbols, stream lengths
    if (lane == 0) *reinterpret_cast<uint4*>(s_out) = make_uint4(1u | (k[pl] << 16), 0, 0, 0);
    uint32_t nib = 0, present = 0;
    for (int r = 0; r < 4; r++) {
      nib |= (f[pl][r] != 0) << r;
      present += f[pl][r] != 0;
    }
    const uint32_t other = __shfl_xor(nib, 1, 64);
    if (!(lane & 1)) s_out[16 + lane / 2] = (uint8_t)(nib | (other << 4));
    uint32_t pos = wave_excl_scan(present);
    for (int r = 0; r < 4; r++)
      if (f[pl][r]) *reinterpret_cast<uint16_t*>(s_out + 48 + 2 * pos++) = (uint16_t)f[pl][r];
    const uint32_t lens = 48 + 2 * k[pl];
    *reinterpret_cast<uint16_t*>(s_out + lens + 2 * lane) = (uint16_t)len[pl];
    const uint32_t st = lens + 2 * kAnsStreams + wave_excl_scan(len[pl]);
    for (uint32_t b = 16 + body[pl] + lane; b < psize[pl]; b += 64) s_out[b] = 0;
    const uint32_t endv[2] = {st + len[pl], st + len[pl]};
    const uint32_t limv[2] = {len[pl] - 4, len[pl] - 4};
    if (pl == 0) {
      if (rawpl == 1) ans_encode_streams<D, true, true, false, 1>(s, n, s_enc, x, cnt, s_out, endv, limv, P1 + 16);
      else ans_encode_streams<D, true, true, false>(s, n, s_enc, x, cnt, s_out, endv, limv);
    } else {
      if (rawpl == 0) ans_encode_streams<D, true, false, true, 0>(s, n, s_enc, x, cnt, s_out, endv, limv, P0 + 16);
      else ans_encode_streams<D, true, false, true>(s, n, s_enc, x, cnt, s_out, endv, limv);
    }
    s_out[st] = (uint8_t)x[pl];                                  // final state, u32 little-endian
    s_out[st + 1] = (uint8_t)(x[pl] >> 8);
    s_out[st + 2] = (uint8_t)(x[pl] >> 16);
    s_out[st + 3] = (uint8_t)(x[pl] >> 24);
    __syncthreads();
    for (uint32_t u = lane; u < psize[pl] / 16; u += 64)
      st_global16(P + 16 * u, *reinterpret_cast<const uint4*>(s_out + 16 * u));
    __syncthreads();                                             // the image is rebuilt for the next plane
  }
  const uint32_t cr = CRC ? crc32_written<64>(heap, payload, ct, p.tables) : 0u;
  // no fence before the header: nothing reads the payload during this
  // launch, and its completion makes every write visible to later work
  if (lane == 0) {
    write_header_desc(s.slot, desc, slot_off, C_ANS, KVC_FLAG_HEAP | crc_flag, KVC_SEG_ENCODED, (int)p.dtype,
                      comp, D, s.n_vec, payload, off, 0, cr);
  }
}

// Whether a coded plane's model (payload bytes P in global memory) is well
// formed: the bitmap holds K symbols, each with a nonzero frequency, and the
// frequencies sum to 4096.
__device__ __forceinline__ bool ans_model_ok(const uint8_t* P, uint32_t k) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t bits = (P[16 + lane / 2] >> (4 * (lane & 1))) & 15u;   // symbols 4 lane .. 4 lane + 3
  const uint32_t present = __popc(bits);
  uint32_t pos = wave_excl_scan(present);
  const bool ok_k = wave_sum(present) == k;
  uint32_t tot = 0;
  bool ok = true;
  for (int r = 0; r < 4; r++)
    if ((bits >> r) & 1) {
      const uint32_t fr = pos < k ? *reinterpret_cast<const uint16_t*>(P + 48 + 2 * pos++) : 0;
      ok = ok && fr != 0;
      tot += fr;
    }
  return __all(ok) && ok_k && wave_sum(tot) == kAnsM;
}

// slot -> symbol table of a well-formed coded plane and its (f, cum) pairs.
// Lane j fills slots [64 j, 64 j + 64), four to a word.
__device__ __forceinline__ void ans_build_tables(const uint8_t* P, uint32_t k, AnsDec* tab, uint8_t* lut) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t bits = (P[16 + lane / 2] >> (4 * (lane & 1))) & 15u;
  uint32_t pos = wave_excl_scan((uint32_t)__popc(bits));
  uint32_t fr[4], tot = 0;
  for (int r = 0; r < 4; r++) {
    fr[r] = (bits >> r) & 1 && pos < k ? *reinterpret_cast<const uint16_t*>(P + 48 + 2 * pos++) : 0;
    tot += fr[r];
  }
  uint32_t run = wave_excl_scan(tot);
  for (int r = 0; r < 4; r++) {
    tab[4 * lane + r] = AnsDec{(uint16_t)fr[r], (uint16_t)run};
    run += fr[r];
  }
  __syncthreads();
  // the symbol of slot 64 lane: the largest with cum <= 64 lane (it has f > 0,
  // since a later symbol with f = 0 would share its cum), then walk
  const uint32_t s0 = 64 * lane;
  uint32_t lo = 0, hi = 255;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (tab[mid].cum <= s0) lo = mid;
    else hi = mid - 1;
  }
  uint32_t sy = lo, lim = (uint32_t)tab[sy].cum + tab[sy].f;
  for (uint32_t w = 0; w < 16; w++) {
    uint32_t word = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4; b++) {
      while (s0 + 4 * w + b >= lim) {                            // frequencies sum to 4096: ends by sy = 255
        sy++;
        lim = (uint32_t)tab[sy].cum + tab[sy].f;
      }
      word |= sy << (8 * b);
    }
    *reinterpret_cast<uint32_t*>(lut + s0 + 4 * w) = word;
  }
  __syncthreads();
}

// 4 payload bytes at aligned offset a, or at the last aligned offset of the
// checked span when a is past it (such bytes lie beyond every stream)
__device__ __forceinline__ uint32_t ans_word(const uint8_t* heap, uint32_t a, uint32_t span) {
  return ld_global4(heap + min(a, span - 4));
}
// the 16 payload bytes at block-aligned offset b, likewise
__device__ __forceinline__ uint4 ans_block(const uint8_t* heap, uint32_t b, uint32_t span) {
  return ld_global16(heap + min(b, span - 16));
}

// A lane's window on its stream of the coded plane: a ring of four 16-byte
// blocks in LDS; word w of lane j at ring[64 w + j] (a bank per lane).  The
// block at payload offset b (a multiple of 16) occupies words (b / 4) mod 16
// to + 3; word 16 repeats word 0, so that the word after any word w < 16 is
// ring[64 (w + 1) + j].
constexpr uint32_t kAnsRingWords = 16;
__device__ __forceinline__ void ans_ring_put(uint32_t* ring, uint32_t b, uint4 v) {
  const uint32_t j = threadIdx.x & 63, w = (b >> 2) & (kAnsRingWords - 1);
  ring[64 * w + j] = v.x;
  ring[64 * (w + 1) + j] = v.y;
  ring[64 * (w + 2) + j] = v.z;
  ring[64 * (w + 3) + j] = v.w;
  if (w == 0) ring[64 * kAnsRingWords + j] = v.x;
}
// the 4 stream bytes from payload offset q, the first in the low byte
__device__ __forceinline__ uint32_t ans_ring_bytes(const uint32_t* ring, uint32_t q) {
  const uint32_t* const r = ring + 64 * ((q >> 2) & (kAnsRingWords - 1)) + (threadIdx.x & 63);
  return __builtin_amdgcn_alignbyte(r[64], r[0], q & 3);
}

// Where the byte of the plane not being decoded comes from
enum AnsOther { kOtherRaw = 0, kOtherZero = 1, kOtherPage = 2 };

// Decode lane j's stream (chunks j, j + 64, ...) of coded plane CP and write
// each chunk of 8 values; the other plane's byte comes from its raw bytes at
// payload offset other + 16 (kOtherRaw), is zero (kOtherZero), or is the
// byte already in the destination page (kOtherPage: written by this lane's
// kOtherZero pass over the other plane).  Returns true when the stream is
// malformed: a state outside [2^23, 2^31) at its start, more bytes consumed
// than it holds, or an end other than exactly its last byte in state 2^23.
//
// The stream's bytes reach the lane through its ring: the ring holds the
// blocks of pos and pos + 16 during a chunk (a chunk consumes at most 16
// bytes: two per value), and the block two ahead is loaded while a chunk is
// decoded and stored into the ring before the next one.  The other plane's
// bytes are likewise loaded a chunk ahead.  A state x >= 2^23 leaves a
// decode step at or above 2^11, so one byte brings it back above 2^23 from
// [2^15, 2^23) and two from [2^11, 2^15).
template <int D, int CP, int OTHER>
__device__ __forceinline__ bool ans_decode_lanes(const SegCtx& s, uint16_t* page_p, const uint8_t* heap, uint32_t span,
                                                 uint32_t chunks, uint32_t other, uint32_t sbeg, uint32_t send,
                                                 const AnsDec* tab, const uint8_t* lut, uint32_t* ring) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t a = sbeg & ~3u;                                 // final state, u32 little-endian
  uint32_t x = __builtin_amdgcn_alignbyte(ans_word(heap, a + 4, span), ans_word(heap, a, span), sbeg & 3);
  bool bad = x < kAnsL || x >= (kAnsL << 8);
  uint32_t pos = sbeg + 4;
  const uint32_t b0 = pos & ~15u;
  ans_ring_put(ring, b0, ans_block(heap, b0, span));
  ans_ring_put(ring, b0 + 16, ans_block(heap, b0 + 16, span));
  uint32_t nb = b0 + 32;
  uint4 pend = ans_block(heap, nb, span);
  uint2 rb = make_uint2(0, 0);
  uint4 pg = make_uint4(0, 0, 0, 0);
  if constexpr (OTHER == kOtherRaw)
    if (lane < chunks) rb = ld_global8(heap + other + 16 + 8 * lane);
  if constexpr (OTHER == kOtherPage)
    if (lane < chunks) pg = ld_global16(byte_at(page_p, 2 * ans_chunk_off(s, lane, D)));
  for (uint32_t c = lane; c < chunks; c += kAnsStreams) {
    ans_ring_put(ring, nb, pend);
    nb = (pos & ~15u) + 32;
    pend = ans_block(heap, nb, span);
    uint32_t ob[8];                                              // the other plane's bytes of this chunk
    if constexpr (OTHER == kOtherRaw) {
      const uint2 r = rb;
      if (c + kAnsStreams < chunks) rb = ld_global8(heap + other + 16 + 8 * (c + kAnsStreams));
#pragma unroll
      for (int e = 0; e < 8; e++) ob[e] = ((e < 4 ? r.x : r.y) >> (8 * (e & 3))) & 0xFFu;
    } else if constexpr (OTHER == kOtherPage) {
      const uint32_t w[4] = {pg.x, pg.y, pg.z, pg.w};
      if (c + kAnsStreams < chunks) pg = ld_global16(byte_at(page_p, 2 * ans_chunk_off(s, c + kAnsStreams, D)));
#pragma unroll
      for (int e = 0; e < 8; e++) ob[e] = (w[e >> 1] >> (16 * (e & 1) + 8 * (1 - CP))) & 0xFFu;
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++) ob[e] = 0;
    }
    uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t q = ans_ring_bytes(ring, pos);             // the next stream bytes b0, b1 in bits 0..15
      const uint32_t sl = x & (kAnsM - 1), sy = lut[sl];
      const AnsDec t = tab[sy];
      x = __umul24(t.f, x >> kAnsProbBits) + sl - t.cum;
      // x < 2^23 takes b0: (x << 8) | b0; x < 2^15 takes b0, b1: (x << 16) |
      // (b0 << 8) | b1 -- byte permutes of x and q (the bytes they drop are 0)
      const bool one = x < kAnsL, two = x < (kAnsL >> 8);
      const uint32_t x1 = __builtin_amdgcn_perm(x, q, 0x06050400u), x2 = __builtin_amdgcn_perm(x, q, 0x05040001u);
      x = two ? x2 : (one ? x1 : x);
      pos += (uint32_t)one + (uint32_t)two;                      // a stream read past its end ends past it
      const uint32_t v = CP ? (sy << 8) | ob[e] : (ob[e] << 8) | sy;
      o[e >> 1] |= v << (16 * (e & 1));
    }
    st_global16(byte_at(page_p, 2 * ans_chunk_off(s, c, D)), make_uint4(o[0], o[1], o[2], o[3]));
  }
  return bad || pos != send || x != kAnsL;                      // pos only grows: a read past send shows here
}

template <int D, bool CRC>
__global__ __launch_bounds__(64) void ans_decode_kernel(CallParams p) {
  __shared__ AnsDec s_tab[256];
  __shared__ __attribute__((aligned(16))) uint8_t s_lut[kAnsM];
  __shared__ uint32_t s_ring[64 * (kAnsRingWords + 1)];
  CrcLds* const ct = crc_tables_lds<CRC>();
  const uint32_t seg = p.seg_base + blockIdx.x;
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry E = side_entry(p, 2 * l + comp);
  if (E.codec != C_ANS) return;
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = page_id(p, pi);
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
  else ok = ok && format == C_ANS && (flags & KVC_FLAG_HEAP) && stored >= 32 && stored <= (1u << 30);
  // every read stays in the buffer: the stored bytes rounded up to 16, from
  // a 16-byte aligned offset (payload offsets are 32-bit: stored <= 2^30 is
  // far above any payload of a segment of at most 32 KiB)
  const uint64_t span = ((uint64_t)stored + 15) & ~15ull;
  ok = ok && (spill & 15) == 0 && spill >= p.slot_region && span <= p.buf_bytes && spill <= p.buf_bytes - span;
  if (!ok) {
    if (report) p.seg_status[seg] = 1;
    return;
  }
  const uint8_t* const heap = p.buf + spill;
  if constexpr (CRC) {
    __syncthreads();                                             // CRC tables in LDS
    if (crc32_lanes<64, kCarryChain>(GlobalBytes{heap}, stored, ct, p.tables) != h1.z) {
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
  // parse both planes' headers, check their models, lengths and padding
  uint32_t pbase[2], mode[2], kk[2], sbeg[2] = {0, 0}, send[2] = {0, 0};
  uint32_t at = 0;
  bool good = true;
  for (int pl = 0; pl < 2 && good; pl++) {
    const uint8_t* const P = heap + at;
    pbase[pl] = at;
    good = at + 16 <= stored;
    if (!good) break;
    const uint4 hd = ld_global16(P);
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
      const uint32_t len = *reinterpret_cast<const uint16_t*>(heap + lens_at + 2 * lane);
      const uint32_t st0 = lens_at + 2 * kAnsStreams + wave_excl_scan(len);
      sbeg[pl] = st0;
      send[pl] = st0 + len;
      good = __all(len >= 4) && wave_max(st0 + len) <= stored;
      size = 48 + 2 * kk[pl] + 2 * kAnsStreams + wave_sum(len);
      if (good) good = ans_model_ok(P, kk[pl]);
    }
    const uint32_t padded = (size + 15) & ~15u;
    good = good && at + padded <= stored;
    if (good) good = __all(lane >= padded - size || heap[at + size + lane] == 0);   // zero padding
    at += padded;
  }
  good = good && at == stored;                                   // exact length of the payload
  if (!good) {
    if (report) p.seg_status[seg] = 1;
    return;
  }
  // one coded plane at a time: its tables and ring in LDS
  const uint32_t span32 = (uint32_t)span;
  bool bad = false;
  if (mode[0] && mode[1]) {                                      // low plane first, then the high merged in
    ans_build_tables(heap + pbase[0], kk[0], s_tab, s_lut);
    bad = ans_decode_lanes<D, 0, kOtherZero>(s, page_p, heap, span32, chunks, 0, sbeg[0], send[0], s_tab, s_lut, s_ring);
    __syncthreads();
    ans_build_tables(heap + pbase[1], kk[1], s_tab, s_lut);
    bad |= ans_decode_lanes<D, 1, kOtherPage>(s, page_p, heap, span32, chunks, 0, sbeg[1], send[1], s_tab, s_lut, s_ring);
  } else if (mode[0]) {
    ans_build_tables(heap + pbase[0], kk[0], s_tab, s_lut);
    bad = ans_decode_lanes<D, 0, kOtherRaw>(s, page_p, heap, span32, chunks, pbase[1], sbeg[0], send[0], s_tab, s_lut, s_ring);
  } else if (mode[1]) {
    ans_build_tables(heap + pbase[1], kk[1], s_tab, s_lut);
    bad = ans_decode_lanes<D, 1, kOtherRaw>(s, page_p, heap, span32, chunks, pbase[0], sbeg[1], send[1], s_tab, s_lut, s_ring);
  } else {                                                       // two raw planes
    for (uint32_t c = lane; c < chunks; c += kAnsStreams) {
      const uint2 lo = ld_global8(heap + pbase[0] + 16 + 8 * c), hi = ld_global8(heap + pbase[1] + 16 + 8 * c);
      const uint4 o = make_uint4(__builtin_amdgcn_perm(hi.x, lo.x, 0x05010400u), __builtin_amdgcn_perm(hi.x, lo.x, 0x07030602u),
                                 __builtin_amdgcn_perm(hi.y, lo.y, 0x05010400u), __builtin_amdgcn_perm(hi.y, lo.y, 0x07030602u));
      st_global16(byte_at(page_p, 2 * ans_chunk_off(s, c, D)), o);
    }
  }
  bad = __any(bad);
  if (report) p.seg_status[seg] = bad ? 1 : 0;
}

template <int D, bool CRC>
void launch_ans_encode_dc(const CallParams& p, uint64_t n, hipStream_t st) {
  hipLaunchKernelGGL((ans_encode_kernel<D, CRC>), dim3((unsigned)n), dim3(64), ans_encode_lds(p.stage_bytes), st, p);
}
template <int D, bool CRC>
void launch_ans_decode_dc(const CallParams& p, uint64_t n, hipStream_t st) {
  hipLaunchKernelGGL((ans_decode_kernel<D, CRC>), dim3((unsigned)n), dim3(64), 0, st, p);
}
