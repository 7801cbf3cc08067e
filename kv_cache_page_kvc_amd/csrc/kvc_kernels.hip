// kvc_kernels.hip -- gfx950 kernels of libkvc: fused page gather + encode +
// store, and load + decode + page scatter, for the codecs described on
//   OrbitKV docs, "KV precision and storage encoding", section "FP8 and
//     TurboQuant" (E4M3FN, TurboQuant K, uniform V, raw fallback),
//   "Building a quantized HiCache for SGLang", section "Building the INT8
//     codec" (per-vector INT8),
//   knlp "Asymmetric KV: methods and results", section "Precision and scaling
//     reference" (FP8 scale rule).
//
// Work decomposition.  One 256-thread workgroup per segment (page, layer,
// component).  A head vector of D elements is held by a group of P lanes, each
// lane owning E = D/P elements as NCH = E/8 chunks of 8 contiguous elements
// (one 16-byte load per chunk):
//     element i = k*8P + 8p + j   (chunk k, lane p of the group, j < 8).
// So WHT stages / reduction levels over element bits 0..2 are in-lane, bits
// 3..3+log2(P)-1 are cross-lane and the chunk bits are in-lane again.  P is
// 2, 4, 8, 16 for D = 32, 64, 128, 256.  Positions map onto lanes so that
// every cross-lane partner is one DPP step away (quad_perm for lane xor 1 and
// xor 2, row_ror:8 for lane xor 8, row_half_mirror for lane xor 7; see
// lane_info).  Each load instruction of a wave reads 16 consecutive bytes
// per lane and whole 128-byte lines of consecutive vectors at D >= 128.
//
// Arithmetic: binary32 with round-to-nearest-even, built with
// -ffp-contract=off; '/' and sqrtf are correctly rounded (HIP default);
// fmaf is used only where the fused single rounding is the defined result.
// Data-dependent raw segments: codes are written speculatively, then the
// workgroup OR-reduces the per-vector gate; a raw segment gets a header with
// RAW_DATA, a zeroed slot body and its bytes in the spill region.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvc_arch.h"
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ geometry
template <int D, int NT = kThreadsSmall>
struct Geo {
  static constexpr int P = lanes_per_vector(D);               // lanes per vector
  static constexpr int LOGP = P == 2 ? 1 : (P == 4 ? 2 : (P == 8 ? 3 : 4));
  static constexpr int E = D / P;                             // elements per lane
  static constexpr int NCH = E / 8;                           // 16-byte chunks per lane
  static constexpr int GPW = 64 / P;                          // groups per wave
  static constexpr int GW = groups_per_workgroup(D, NT);      // groups per workgroup
  static_assert(GW == GPW * (NT / 64), "group geometry");
  // vectors per group whose loads are in flight together: 2 keeps the encode
  // kernel at <= 80 VGPRs for D <= 128 (six waves per SIMD), and more vectors
  // per batch measured slower through the lost occupancy
  static constexpr int U = kBatchVectors;
};

// 16-byte units each thread has in flight while it copies a slot or a table
// into LDS: all its loads are issued before the first store
constexpr int kStageRounds = 4;

struct Lane {
  int p;        // lane index within the group
  int g;        // group index within the workgroup
};

// Group position p -> lane within the group's lanes: a linear map over
// GF(2) that sends position bit q to the lane mask of the q-th cross-lane
// partner (1, 2, 8 and, for 16-lane groups, 7): position p and p ^ (1 << q)
// then sit in lanes l and l ^ mask(q), one DPP step apart (quad_perm for 1
// and 2, row_ror:8 for 8, row_half_mirror for 7).  The inverse below gives p
// from the lane id.
template <int D>
__device__ __forceinline__ Lane lane_info() {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Lane r;
  if constexpr (Geo<D>::P == 16) {
    const int l = lane & 15, b2 = (l >> 2) & 1;        // lane bit 2 = position bit 3
    r.p = ((l & 1) ^ b2) | ((((l >> 1) & 1) ^ b2) << 1) | (((l >> 3) & 1) << 2) | (b2 << 3);
    r.g = wave * 4 + (lane >> 4);
  } else if constexpr (Geo<D>::P == 8) {
    r.p = (lane & 3) | (((lane >> 3) & 1) << 2);
    r.g = wave * 8 + (((lane >> 2) & 1) | ((lane >> 4) << 1));
  } else if constexpr (Geo<D>::P == 4) {
    r.p = lane & 3;
    r.g = wave * 16 + (lane >> 2);
  } else {
    r.p = lane & 1;
    r.g = wave * 32 + (lane >> 1);
  }
  return r;
}

// cross-lane partner for the q-th group bit (element bit 3+q): DPP control
// quad_perm:[1,0,3,2] (lane ^ 1), quad_perm:[2,3,0,1] (lane ^ 2), row_ror:8
// (lane ^ 8), row_half_mirror (lane ^ 7)
template <int Q>
constexpr int xlane_ctrl() { return Q == 0 ? 0xB1 : (Q == 1 ? 0x4E : (Q == 2 ? 0x128 : 0x141)); }
template <int Q>
__device__ __forceinline__ float xlane(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), xlane_ctrl<Q>(), 0xF, 0xF, true));
}
template <int Q>
__device__ __forceinline__ uint32_t xlane_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, xlane_ctrl<Q>(), 0xF, 0xF, true);
}

// xor of x over the 64 lanes of the wave: over each row of 16 lanes by DPP
// (partners lane ^ 1, ^ 2, ^ 7, ^ 8), then the four rows' results
__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
  x ^= xlane_u<0>(x);
  x ^= xlane_u<1>(x);
  x ^= xlane_u<3>(x);
  x ^= xlane_u<2>(x);
  return (uint32_t)(__builtin_amdgcn_readlane((int)x, 0) ^ __builtin_amdgcn_readlane((int)x, 16) ^
                    __builtin_amdgcn_readlane((int)x, 32) ^ __builtin_amdgcn_readlane((int)x, 48));
}

template <int LOGP>
__device__ __forceinline__ float group_sum(float v) {   // sum over element bits 3.. (ascending)
  if constexpr (LOGP >= 1) v = v + xlane<0>(v);
  if constexpr (LOGP >= 2) v = v + xlane<1>(v);
  if constexpr (LOGP >= 3) v = v + xlane<2>(v);
  if constexpr (LOGP >= 4) v = v + xlane<3>(v);
  return v;
}
template <int LOGP>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  if constexpr (LOGP >= 1) v = max(v, xlane_u<0>(v));
  if constexpr (LOGP >= 2) v = max(v, xlane_u<1>(v));
  if constexpr (LOGP >= 3) v = max(v, xlane_u<2>(v));
  if constexpr (LOGP >= 4) v = max(v, xlane_u<3>(v));
  return v;
}

// ------------------------------------------------------------------ formats
template <int DT>
__device__ __forceinline__ void unpack8(const uint4& w, float* x) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int m = 0; m < 4; m++) {
    if constexpr (DT == KVC_BF16) {
      x[2 * m] = __uint_as_float(a[m] << 16);
      x[2 * m + 1] = __uint_as_float(a[m] & 0xFFFF0000u);
    } else {
      f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, a[m]), f32x2);
      x[2 * m] = f.x;
      x[2 * m + 1] = f.y;
    }
  }
}

// two floats -> packed output pair, round to nearest even
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2 v = {a, b};
  if constexpr (DT == KVC_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

template <int DT>
__device__ __forceinline__ uint4 pack8(const float* y) {
  uint4 w;
  w.x = pack2<DT>(y[0], y[1]);
  w.y = pack2<DT>(y[2], y[3]);
  w.z = pack2<DT>(y[4], y[5]);
  w.w = pack2<DT>(y[6], y[7]);
  return w;
}

// largest |x| bit pattern (sign cleared) of the lane's elements: orders like
// |x| for finite values, and any NaN/Inf pattern is above every finite one.
__device__ __forceinline__ uint32_t absmax_bits(const uint4& w) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) m = max(m, max(a[q] & 0x7FFFu, (a[q] >> 16) & 0x7FFFu));
  return m;
}
template <int DT>
__device__ __forceinline__ float bits_to_f32(uint32_t h) {
  if constexpr (DT == KVC_BF16) return __uint_as_float(h << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <int DT> struct Lim {
  static constexpr uint32_t nonfinite = DT == KVC_BF16 ? 0x7F80u : 0x7C00u;  // |x| bits >= : NaN/Inf
  static constexpr uint32_t fp8max = DT == KVC_BF16 ? 0x43E0u : 0x5F00u;     // 448
};

__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// FP8 E4M3FN (OCP) pack of 8 values (gfx950 v_cvt_pk_fp8_f32: RNE)
__device__ __forceinline__ uint2 fp8x8(const float* q) {
  uint2 r;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  r.x = (uint32_t)lo;
  r.y = (uint32_t)hi;
  return r;
}

// RN(a / N) for a >= 0 (or +Inf/NaN, which stay non-finite) from the
// constant RN(1/N) and one FMA residual step: q0 = RN(a*r), e = a - N*q0
// (exact), RN(q0 + e*r).  Checked against the IEEE quotient for every
// non-negative binary32 a, for N = 7, 15 and 127.
template <int N>
__device__ __forceinline__ float div_const(float a) {
  static_assert(N == 7 || N == 15 || N == 127, "verified divisors only");
  constexpr float r = 1.0f / (float)N;
  const float q0 = a * r;
  return fmaf(fmaf(-q0, (float)N, a), r, q0);
}

// x / s for a vector's scale s, from r = RN(1/s): q0 = RN(x*r), e = x - s*q0
// (exact), RN(q0 + e*r).  For every scale the INT8, INT8 record and FP8
// dynamic codecs form and every |x| <= the vector's amax (BF16 and FP16
// sources, all checked exhaustively), the stored code is the one the IEEE
// quotient gives: FP16 quotients are identical, BF16 ones differ only
// below 2^-10, which both codes map to zero.
__device__ __forceinline__ float div_scaled(float x, float s, float r) {
  const float q0 = x * r;
  return fmaf(fmaf(-q0, s, x), r, q0);
}

// Uniform code of d = RN(x - m_h) against the FP16 scale s = sigma_h, as
// the bits of RN(q + 1.5*2^23) with q = RN(d / s): for |q| < 2^22 these are
// 0x4B400000 + RNE(q), and clamping them as integers to [0x4B400000,
// 0x4B400000 + 2^b - 1] gives clamp(RNE(q), 0, 2^b - 1) for every q.  The
// quotient comes from y = RN(1/s): q0 = RN(d*y), then one FMA residual step
// RN(q0 + RN(d - q0*s)*y), which equals RN(d / s) for every positive finite
// FP16 s and every d >= s/4 (checked over every pair of significands; for
// smaller d both codes are 0).  With s == 0 (y == 0) q is 0 for finite d.
__device__ __forceinline__ int uniform_code_bits(float d, float s, float y) {
  const float q0 = d * y;
  const float q = fmaf(fmaf(-q0, s, d), y, q0);
  return __float_as_int(q + 12582912.0f);
}

// ------------------------------------------------------------------ addressing
struct SegCtx {
  const uint16_t* src;      // element (t=0, h=0, i=0) of the page's component
  uint8_t* slot;            // slot start (header)
  int n_vec;
  int heads;
  uint64_t heads_magic;     // v / heads = (v * heads_magic) >> 32 for v < 2^16
  uint32_t st, sh;          // element strides of token and head
  uint32_t walk_dh, walk_step, walk_wrap;
  uint32_t linear_iters;    // batches per group of a linear layout, else 0
  uint32_t row_bytes;       // record codec: bytes of one token row
};

// A lane's current vector: its head and its element offset in the page
// (below 2^31, checked on the host).
struct VecPos {
  int h;
  uint32_t off;
};

__device__ __forceinline__ VecPos vec_pos(const SegCtx& s, int v) {
  const int t = (int)(((uint64_t)(uint32_t)v * s.heads_magic) >> 32), h = v - t * s.heads;
  VecPos q;
  q.h = h;
  q.off = (uint32_t)t * s.st + (uint32_t)h * s.sh;
  return q;
}
// from vector v to v + GW: the head advances by GW mod heads, with a carry
// into the token
__device__ __forceinline__ void vec_advance(const SegCtx& s, VecPos& q) {
  q.h += (int)s.walk_dh;
  q.off += s.walk_step;
  if (q.h >= s.heads) {
    q.h -= s.heads;
    q.off += s.walk_wrap;
  }
}
// base + a 32-bit byte offset (global_load/store with a scalar base)
template <class T>
__device__ __forceinline__ T* byte_at(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}
template <class T>
__device__ __forceinline__ const T* byte_at(const T* base, uint32_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

// The call's side-table entry idx and page id i: from the kernel arguments
// for a small call, else from the table the host uploaded.  Both are read
// through the constant address space, so the loads stay scalar.
typedef const __attribute__((address_space(4))) uint64_t ConstU64;
typedef const __attribute__((address_space(4))) int32_t ConstI32;
__device__ __forceinline__ SideEntry side_entry(const CallParams& p, uint32_t idx) {
  static_assert(sizeof(SideEntry) == 4 * sizeof(uint64_t), "a side entry is four 8-byte words");
  ConstU64* t = p.inline_tables ? (ConstU64*)&p.sides_inline[0] : (ConstU64*)p.sides;
  uint64_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) w[i] = t[4 * idx + i];
  SideEntry e;
  __builtin_memcpy(&e, w, sizeof(e));
  return e;
}
__device__ __forceinline__ int32_t page_id(const CallParams& p, uint32_t i) {
  ConstI32* t = p.inline_tables ? (ConstI32*)&p.pages_inline[0] : (ConstI32*)p.pages;
  return t[i];
}

// Reserve `need` bytes of the spill region: the offset of the reservation.
// A cursor with a lap tag holds the lap in its high bits; the call's first
// reservation replaces a value from an earlier lap, the others add to it.
__device__ __forceinline__ uint64_t spill_reserve(const CallParams& p, uint64_t need) {
  if (p.cursor_lap == 0) return atomicAdd(p.spill_cursor, (unsigned long long)need);
  const unsigned long long tag = (unsigned long long)p.cursor_lap << kCursorLapShift;
  unsigned long long cur = *reinterpret_cast<volatile unsigned long long*>(p.spill_cursor);
  for (;;) {
    const bool mine = (cur >> kCursorLapShift) == p.cursor_lap;
    const unsigned long long next = mine ? cur + need : tag + need;
    const unsigned long long prev = atomicCAS(p.spill_cursor, cur, next);
    if (prev == cur) return mine ? cur - tag : 0ull;
    cur = prev;
  }
}

// ------------------------------------------------------------------ encoders
// Each returns 1 if this vector forces the segment raw.
enum Codec { C_RAW = 0, C_FP8D = 1, C_FP8F = 2, C_FP8Y = 3, C_INT8 = 4, C_U3 = 5, C_U4 = 6, C_TQ3 = 7, C_TQ4 = 8,
             C_I8R = 9, C_ANS = 10 };

template <int C> struct CodecInfo {
  static constexpr int bits = (C == C_U3 || C == C_TQ3) ? 3 : ((C == C_U4 || C == C_TQ4) ? 4 : 8);
  static constexpr int meta = (C == C_FP8Y || C == C_INT8 || C == C_U3 || C == C_U4) ? 4
                            : ((C == C_TQ3 || C == C_TQ4 || C == C_I8R) ? 2 : 0);
  static constexpr bool rows = C == C_I8R;       // token-row record layout
  static constexpr bool tq = C == C_TQ3 || C == C_TQ4;
  static constexpr bool uni = C == C_U3 || C == C_U4;
  static constexpr bool fp8 = C == C_FP8D || C == C_FP8F || C == C_FP8Y;
};

// Per-lane sign masks for TurboQuant: flip[4k+m] is the XOR mask of the
// lane's m-th packed 16-bit pair of chunk k -- bit 15 for its element 2m,
// bit 31 for element 2m+1 (the sign-bit positions of BF16 and FP16 pairs).
template <int D>
struct LaneSigns {
  uint32_t flip[Geo<D>::NCH * 4];
};

// sigma_i for the lane's elements, read from the D-bit mask (bit i set:
// sigma_i = -1).  With `parity`, every element of a lane whose position in
// its group has odd bit parity is flipped once more: the cross-lane
// butterflies then reduce to own + partner in both lanes (see wht_cross).
template <int D>
__device__ __forceinline__ void make_lane_signs(const uint32_t* mask, int p, bool parity, LaneSigns<D>& ls) {
  constexpr int P = Geo<D>::P, NCH = Geo<D>::NCH;
  const uint32_t par = (parity && (__builtin_popcount(p) & 1)) ? 0xFFu : 0u;
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    const int e0 = k * 8 * P + 8 * p;            // multiple of 8: one byte of the mask
    const uint32_t byte = ((mask[e0 >> 5] >> (e0 & 31)) & 0xFFu) ^ par;
    // spread holds bit j of the byte at bits j and j + 15; shifted left by
    // 15 - 2m, bit 15 then holds bit 2m and bit 31 bit 2m + 1
    const uint32_t spread = byte | (byte << 15);
#pragma unroll
    for (int m = 0; m < 4; m++) ls.flip[4 * k + m] = (spread << (15 - 2 * m)) & 0x80008000u;
  }
}

// Cross-lane WHT stages.  Stage q pairs lanes whose group position differs
// in bit q; the lower lane needs RN(a+b), the upper RN(a-b).  Every value
// enters with the lane's sign (-1)^parity(position) already applied, so a
// lower lane holds pi*a and sees -pi*b, an upper lane holds -pi*b and sees
// pi*a.  Both then compute one FMA with a +-1 multiplier, own + c*partner
// (c = -1 in the lower lane, +1 in the upper): pi*RN(a+b) and pi*RN(a-b),
// a single rounding because c*partner is exact.  Each stage removes one
// parity bit from the sign, so after the last stage every sign is +1.
// p: the lane's position in its group; its bit q says upper or lower.
template <int LOGP, int E>
__device__ __forceinline__ void wht_cross(float* y, int p) {
  static_assert(E % 8 == 0, "lanes hold whole 8-element chunks");
  if constexpr (LOGP >= 1) {
    const float c = (p & 1) ? 1.0f : -1.0f;
#pragma unroll
    for (int e = 0; e < E; e += 8) fmac_xlane8<0>(y + e, c);
  }
  if constexpr (LOGP >= 2) {
    const float c = (p & 2) ? 1.0f : -1.0f;
#pragma unroll
    for (int e = 0; e < E; e += 8) fmac_xlane8<1>(y + e, c);
  }
  if constexpr (LOGP >= 3) {
    const float c = (p & 4) ? 1.0f : -1.0f;
#pragma unroll
    for (int e = 0; e < E; e += 8) fmac_xlane8<2>(y + e, c);
  }
  if constexpr (LOGP >= 4) {
    const float c = (p & 8) ? 1.0f : -1.0f;
#pragma unroll
    for (int e = 0; e < E; e += 8) fmac_xlane8<3>(y + e, c);
  }
}

// in-lane WHT stages over element bits 0..2 (within each chunk)
template <int NCH>
__device__ __forceinline__ void wht_inlane_low(float* y) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int k = 0; k < NCH; k++)
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (!(j & h)) {
          const float a = y[8 * k + j], b = y[8 * k + j + h];
          y[8 * k + j] = a + b;
          y[8 * k + j + h] = a - b;
        }
}
// in-lane WHT stages over the chunk bits (element bits above the group bits)
template <int NCH>
__device__ __forceinline__ void wht_inlane_high(float* y) {
#pragma unroll
  for (int kh = 1; kh < NCH; kh <<= 1)
#pragma unroll
    for (int k = 0; k < NCH; k++)
      if (!(k & kh))
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const float a = y[8 * k + j], b = y[8 * (k + kh) + j];
          y[8 * k + j] = a + b;
          y[8 * (k + kh) + j] = a - b;
        }
}

// pairwise sum of squares in element-index order: in-lane over bits 0..2,
// cross-lane over the group bits, then in-lane over the chunk bits
template <int NCH, int LOGP>
__device__ __forceinline__ float sumsq_tree(const float* y) {
  float part[NCH];
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; j++) s[j] = y[8 * k + j] * y[8 * k + j];
#pragma unroll
    for (int wdt = 8; wdt > 1; wdt >>= 1)
#pragma unroll
      for (int j = 0; j < wdt / 2; j++) s[j] = s[2 * j] + s[2 * j + 1];
    part[k] = group_sum<LOGP>(s[0]);
  }
#pragma unroll
  for (int wdt = NCH; wdt > 1; wdt >>= 1)
#pragma unroll
    for (int k = 0; k < wdt / 2; k++) part[k] = part[2 * k] + part[2 * k + 1];
  return part[0];
}

// store the codes of one chunk (8 elements) of a vector's code block
// The stores below go to an image of the slot: the LDS stage when the slot is
// assembled there, else the output slot itself (the caller's pointer decides).
template <int D, int BITS>
__device__ __forceinline__ void store_codes(uint8_t* slot, uint32_t cv, int k, int p, uint32_t lo, uint32_t hi) {
  constexpr int P = Geo<D>::P;
  const uint32_t e0 = k * 8 * P + 8 * p;            // first element of the chunk
  if constexpr (BITS == 8) {
    *byte_at(reinterpret_cast<uint2*>(slot), cv + e0) = make_uint2(lo, hi);
  } else if constexpr (BITS == 4) {
    *byte_at(reinterpret_cast<uint32_t*>(slot), cv + e0 / 2) = lo;
  } else {                                          // 3 bits: 24-bit piece at byte 3*e0/8
    uint8_t* q = byte_at(slot, cv + (3 * e0) / 8);  // any byte alignment
    q[0] = (uint8_t)lo;
    q[1] = (uint8_t)(lo >> 8);
    q[2] = (uint8_t)(lo >> 16);
  }
}

// sum over j of (MAGIC << BITS*j), modulo 2^32: the uniform codes are
// accumulated as raw FMA result bits MAGIC + code and corrected once
template <int BITS>
__device__ __forceinline__ constexpr uint32_t magic_sum() {
  uint32_t s = 0;
  for (int j = 0; j < 8; j++) s += 0x4B400000u << (BITS * j);
  return s;
}

// Byte offsets in the slot of vector v's codes (cv) and metadata (mv):
// after the header, the codes block then the metadata block; for the record
// codec, in token row v / heads from kRowsOffset, the codes of head v % heads
// then, after all the row's codes, its BF16 scale.
template <int D, int C>
__device__ __forceinline__ void vec_offsets(const SegCtx& s, int v, uint32_t meta_blk, uint32_t& cv, uint32_t& mv) {
  if constexpr (CodecInfo<C>::rows) {
    const uint32_t t = (uint32_t)(((uint64_t)(uint32_t)v * s.heads_magic) >> 32), h = (uint32_t)v - t * s.heads;
    const uint32_t row = kRowsOffset + t * s.row_bytes;
    cv = row + h * D;
    mv = row + (uint32_t)s.heads * D + 2 * h;
  } else {
    cv = kHeaderBytes + (uint32_t)v * (CodecInfo<C>::bits * D / 8);
    mv = meta_blk + (uint32_t)v * CodecInfo<C>::meta;
  }
}

// TurboQuant codes of a lane's transformed values y: cell c = RNE(4z) + 64
// of the threshold table, code = base(c) + (z > T(c)).  The caller keeps
// |z| < 16.125, so c lies in [0, 128].
template <int D, int BITS>
__device__ __forceinline__ void tq_bucketize(const float* y, const CellEntry* cells, uint8_t* slot, uint32_t cv,
                                             int p) {
  constexpr int NCH = Geo<D>::NCH;
  constexpr int LO = 0x4B400000 - kCellOffset;
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    uint32_t acc = 0;                    // element j ends up at bits [BITS*j, BITS*j + BITS)
#pragma unroll
    for (int j = 7; j >= 0; j--) {
      const float z = y[8 * k + j];
      const int t = __float_as_int(fmaf(z, kCellScale, 12582912.0f));
      const int idx = t - LO;
      const CellEntry ce = cells[idx];
      acc = (acc << BITS) + ce.base + (z > ce.thr ? 1u : 0u);
    }
    store_codes<D, BITS>(slot, cv, k, p, acc, 0);
  }
}

template <int D, int DT, int C>
__device__ __forceinline__ int encode_vector(uint4* w, uint32_t cv, uint32_t mv, const Lane& ln, uint8_t* slot,
                                             float fixed, const LaneSigns<D>& ls, const CellEntry* cells) {
  constexpr int E = Geo<D>::E, NCH = Geo<D>::NCH, LOGP = Geo<D>::LOGP;
  constexpr int BITS = CodecInfo<C>::bits;
  if constexpr (CodecInfo<C>::tq) {
    // sigma (and the lane parity sign) applied to the packed source words
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      w[k].x ^= ls.flip[4 * k];
      w[k].y ^= ls.flip[4 * k + 1];
      w[k].z ^= ls.flip[4 * k + 2];
      w[k].w ^= ls.flip[4 * k + 3];
    }
  }
  float x[E];
#pragma unroll
  for (int k = 0; k < NCH; k++) unpack8<DT>(w[k], x + 8 * k);
  int bad = 0;

  if constexpr (CodecInfo<C>::fp8 || C == C_INT8 || C == C_I8R) {
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < NCH; k++) am = max(am, absmax_bits(w[k]));
    am = group_umax<LOGP>(am);
    bad = CodecInfo<C>::fp8 ? (am > Lim<DT>::fp8max) : (am >= Lim<DT>::nonfinite);
    float s = 1.0f;
    if constexpr (C == C_FP8F) s = fixed;
    if constexpr (C == C_FP8Y) {
      const float r448 = 1.0f / 448.0f;
      s = fmaxf(bits_to_f32<DT>(am), 1e-12f) * r448;
    }
    if constexpr (C == C_INT8) s = div_const<127>(fmaxf(bits_to_f32<DT>(am), 1e-12f));
    // record codec: floor and scale are BF16 values; RN(a/127) is rounded to
    // binary32 first, then to BF16
    if constexpr (C == C_I8R)
      s = bf16_round(materialize_f32(div_const<127>(fmaxf(bits_to_f32<DT>(am), bf16_round(1e-12f)))));
    // per-vector scales divide through RN(1/s); so does the caller's fixed
    // scale within [2^-60, 2^60], where the shortcut is the IEEE quotient
    // (outside, only the IEEE division is used)
    const float rs = C == C_FP8Y || C == C_INT8 || C == C_I8R || C == C_FP8F ? 1.0f / s : 0.0f;
    const bool fixed_short = C == C_FP8F && s >= 0x1p-60f && s <= 0x1p60f;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      uint32_t lo, hi;
      if constexpr (C == C_INT8 || C == C_I8R) {
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          float q = rintf(div_scaled(x[8 * k + j], s, rs));
          q = fminf(fmaxf(q, -127.0f), 127.0f);
          b[j] = (uint32_t)(int)q & 0xFFu;
        }
        lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
      } else {
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          float t = x[8 * k + j];
          if constexpr (C == C_FP8Y) t = div_scaled(t, s, rs);
          if constexpr (C == C_FP8F) t = fixed_short ? div_scaled(t, s, rs) : t / s;
          if constexpr (C != C_FP8D) t = fminf(fmaxf(t, -448.0f), 448.0f);
          q[j] = t;
        }
        const uint2 r = fp8x8(q);
        lo = r.x;
        hi = r.y;
      }
      store_codes<D, 8>(slot, cv, k, ln.p, lo, hi);
    }
    if constexpr (C == C_FP8Y || C == C_INT8)
      if (ln.p == 0) *byte_at(reinterpret_cast<float*>(slot), mv) = s;
    if constexpr (C == C_I8R)
      if (ln.p == 0) *byte_at(reinterpret_cast<uint16_t*>(slot), mv) = (uint16_t)(__float_as_uint(s) >> 16);
  }

  if constexpr (CodecInfo<C>::uni) {
    constexpr int TOP = (1 << BITS) - 1;
    // the lane's extremes by IEEE minimum/maximum, which return NaN when
    // any element is NaN; the group's by the hardware min/max, which skip a
    // NaN partner (a lane's own NaN already sends the segment raw)
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < E; e++) {
      mn = __builtin_elementwise_minimum(mn, x[e]);
      mx = __builtin_elementwise_maximum(mx, x[e]);
    }
    const bool lane_nan = mn != mn;
    group_minmax_dpp<LOGP>(mn, mx);
    mn = mn + 0.0f;                      // a zero extreme is +0, whichever zeros the vector holds
    mx = mx + 0.0f;
    const float sig = materialize_f32(div_const<TOP>(mx - mn));   // RN to binary32, then to FP16
    const float mh = f16_round(mn), sh = f16_round(sig);
    // +-Inf reach mn/mx and overflow the FP16 metadata
    bad = lane_nan || !__builtin_isfinite(mh) || !__builtin_isfinite(sh);
    const float y = sh == 0.0f ? 0.0f : recip_newton(sh);
    constexpr int MAGIC = 0x4B400000;   // bits of 1.5 * 2^23
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      uint32_t acc = 0;                  // sum over j of (MAGIC + code_j) << BITS*j
#pragma unroll
      for (int j = 7; j >= 0; j--) {
        const int t = uniform_code_bits(x[8 * k + j] - mh, sh, y);
        acc = (acc << BITS) + (uint32_t)min(max(t, MAGIC), MAGIC + TOP);
      }
      store_codes<D, BITS>(slot, cv, k, ln.p, acc - magic_sum<BITS>(), 0);
    }
    if (ln.p == 0) *byte_at(reinterpret_cast<uint32_t*>(slot), mv) = f16_bits(mh) | (f16_bits(sh) << 16);
  }

  if constexpr (CodecInfo<C>::tq) {
    // 1. norm (signs do not change the squares).  The common case is taken
    // for the whole wave when every active lane's sum of squares S lies in
    // [2^-96, 2^31): then RN(sqrt(S)) and RN(1/n) come from the short
    // sequences (n >= 2^-48), n < 2^15.5 rounds to a finite FP16 value, and
    // every transformed value satisfies |z| <= sqrt(D) (1 + 2^-20) < 16.125
    // (the squares lost to underflow weigh at most 2^-46 of S, each rounding
    // of the sum, the root, the reciprocal, the products and the butterflies
    // at most 2^-24), so its cell index lies in the table without a clamp.
    // Other vectors (zero, tiny, huge or non-finite) take the general path.
    const float S = sumsq_tree<NCH, LOGP>(x);
    const bool common = __builtin_amdgcn_ballot_w64(!(S >= 0x1p-96f && S < 0x1p31f)) == 0;
    float n, r;
    if (common) {
      n = sqrt_rn_normal(S);
      r = recip_newton(n);
    } else {
      n = sqrtf(S);
      bad = !__builtin_isfinite(f16_round(n));
      r = (n == 0.0f || bad) ? 0.0f : 1.0f / n;
    }
    const float nh = f16_round(n);
    // 2.-3. normalise the signed values
    float y[E];
#pragma unroll
    for (int e = 0; e < E; e++) y[e] = x[e] * r;
    // 4. WHT, stages in ascending span
    wht_inlane_low<NCH>(y);
    wht_cross<LOGP, E>(y, ln.p);
    wht_inlane_high<NCH>(y);
    // 5. bucketize: code = #{B_k < z} = base(cell) + (z > T(cell)).  Outside
    // the common case |z| may exceed 16 (or z be NaN, in a vector that sends
    // its segment raw); the edge cells hold no threshold, so clamping z to
    // +-16 (NaN to -16) keeps every cell index in the table and leaves every
    // code as it is.
    if (!common) {
#pragma unroll
      for (int e = 0; e < E; e++) y[e] = fabsf(y[e]) <= 16.0f ? y[e] : (y[e] > 0.0f ? 16.0f : -16.0f);
    }
    tq_bucketize<D, BITS>(y, cells, slot, cv, ln.p);
    if (ln.p == 0) *byte_at(reinterpret_cast<uint16_t*>(slot), mv) = (uint16_t)f16_bits(nh);
  }
  return bad;
}

// the source chunks of vectors v0 + u*GW (u < U) that this lane holds; pos
// is the lane's position at v0 and ends at v0 + U*GW
template <int D, int NT>
__device__ __forceinline__ void load_batch(const SegCtx& s, const Lane& ln, int v0, VecPos& pos,
                                           uint4 (&w)[Geo<D>::U][Geo<D>::NCH]) {
  constexpr int P = Geo<D>::P, NCH = Geo<D>::NCH, GW = Geo<D, NT>::GW, U = Geo<D>::U;
#pragma unroll
  for (int u = 0; u < U; u++) {
    if (v0 + u * GW < s.n_vec) {
      const uint32_t b = 2 * (pos.off + 8 * ln.p);
#pragma unroll
      for (int k = 0; k < NCH; k++) w[u][k] = ld_stream16(byte_at(s.src, b + 16 * P * k));
    }
    vec_advance(s, pos);
  }
}

// Encode the segment's vectors.  Returns nonzero if any vector forces the
// segment raw.
template <int D, int DT, int C, int NT>
__device__ __forceinline__ int encode_segment_vectors(const SegCtx& s, const Lane& ln, float fixed,
                                                      const LaneSigns<D>& ls, const CellEntry* cells,
                                                      uint8_t* image) {
  constexpr int GW = Geo<D, NT>::GW, U = Geo<D>::U;
  constexpr int CB = CodecInfo<C>::bits * D / 8;
  const uint32_t meta_blk = kHeaderBytes + (uint32_t)s.n_vec * CB;   // byte offset in the slot
  int bad = 0;
  uint4 w[U][Geo<D>::NCH];
  if (s.linear_iters) {
    // vector v at element v * D, every batch full: a uniform trip count and
    // one address step per batch
    constexpr int P = Geo<D>::P, NCH = Geo<D>::NCH;
#pragma unroll 1
    for (uint32_t it = 0; it < s.linear_iters; it++) {
      const int v0 = ln.g + (int)it * (GW * U);
#pragma unroll
      for (int u = 0; u < U; u++) {
        const uint32_t b = 2u * ((uint32_t)(v0 + u * GW) * D + 8 * ln.p);
#pragma unroll
        for (int k = 0; k < NCH; k++) w[u][k] = ld_stream16(byte_at(s.src, b + 16 * P * k));
      }
      // (the bound always holds here; as a branch it keeps the vectors'
      // arithmetic apart, which holds the register count of the general loop)
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (v0 + u * GW < s.n_vec) {
          uint32_t cv, mv;
          vec_offsets<D, C>(s, v0 + u * GW, meta_blk, cv, mv);
          bad |= encode_vector<D, DT, C>(w[u], cv, mv, ln, image, fixed, ls, cells);
        }
      }
    }
    return bad;
  }
  VecPos pos = vec_pos(s, ln.g);
  for (int v0 = ln.g; v0 < s.n_vec; v0 += GW * U) {
    load_batch<D, NT>(s, ln, v0, pos, w);
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int v = v0 + u * GW;
      if (v < s.n_vec) {
        uint32_t cv, mv;
        vec_offsets<D, C>(s, v, meta_blk, cv, mv);
        bad |= encode_vector<D, DT, C>(w[u], cv, mv, ln, image, fixed, ls, cells);
      }
    }
  }
  return bad;
}

// copy n bytes (a multiple of 16) from src to dst: a raw slot body to a page
// stored in canonical order (vector v at element v * D).  Every thread has
// kFlatRounds 16-byte units in flight before its first store.
constexpr int kFlatRounds = 8;
template <int NT>
__device__ __forceinline__ void copy_flat(const uint8_t* src, uint8_t* dst, uint32_t n) {
  const uint32_t units = n >> 4;
  for (uint32_t u0 = threadIdx.x; u0 < units; u0 += kFlatRounds * NT) {
    uint4 w[kFlatRounds];
#pragma unroll
    for (int r = 0; r < kFlatRounds; r++)
      w[r] = u0 + r * NT < units ? ld_stream16(src + 16 * (u0 + r * NT)) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < kFlatRounds; r++)
      if (u0 + r * NT < units) st_global16(dst + 16 * (u0 + r * NT), w[r]);
  }
}

// copy a segment from the engine layout into contiguous canonical order; STREAM:
// nontemporal stores, for a destination whose lines each store covers whole
// (the 256-byte aligned spill copies; a slot body starts 32 bytes into a line)
template <int D, int NT, bool STREAM>
__device__ __forceinline__ void copy_out_raw(const SegCtx& s, const Lane& ln, uint8_t* dst) {
  constexpr int P = Geo<D>::P, NCH = Geo<D>::NCH, GW = Geo<D, NT>::GW, U = Geo<D>::U;
  uint4 w[U][NCH];
  VecPos pos = vec_pos(s, ln.g);
  for (int v0 = ln.g; v0 < s.n_vec; v0 += GW * U) {
    load_batch<D, NT>(s, ln, v0, pos, w);
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int v = v0 + u * GW;
      if (v < s.n_vec) {
        const uint32_t b = (uint32_t)v * (2 * D) + 16 * ln.p;
#pragma unroll
        for (int k = 0; k < NCH; k++) {
          if constexpr (STREAM) st_stream16(byte_at(dst, b + 16 * P * k), w[u][k]);
          else st_global16(byte_at(dst, b + 16 * P * k), w[u][k]);
        }
      }
    }
  }
}

// zero bytes [from, to) of a slot; from is even (headers and payloads have
// even sizes) and the padding is shorter than one 256-byte slot unit
template <int NT>
__device__ __forceinline__ void zero_pad(uint8_t* slot, uint32_t from, uint32_t to) {
  for (uint32_t b = from + 2 * threadIdx.x; b < to; b += 2 * NT) *byte_at(reinterpret_cast<uint16_t*>(slot), b) = 0;
}

// zero the bytes of a record-codec slot that no vector writes: the gap
// [32, kRowsOffset) after the header, each token row's padding after its
// codes and scales, and the slot's tail after the last row
template <int NT>
__device__ __forceinline__ void zero_row_gaps(uint8_t* slot, uint32_t tokens, uint32_t heads, uint32_t d,
                                              uint32_t row_bytes, uint32_t slot_bytes) {
  zero_pad<NT>(slot, kHeaderBytes, kRowsOffset);
  const uint32_t used = heads * (d + 2), pad_half = (row_bytes - used) / 2;   // used is even
  for (uint32_t i = threadIdx.x; i < tokens * pad_half; i += NT) {
    const uint32_t t = i / pad_half, j = i - t * pad_half;
    *byte_at(reinterpret_cast<uint16_t*>(slot), kRowsOffset + t * row_bytes + used + 2 * j) = 0;
  }
  zero_pad<NT>(slot, kRowsOffset + tokens * row_bytes, slot_bytes);
}

// the two 16-byte words of a slot header
struct Header {
  uint4 h0, h1;
};
__device__ __forceinline__ Header make_header(int format, int flags, int dtype, int comp, int d, int n_vec,
                                              uint32_t stored, uint64_t spill, uint32_t aux, uint32_t crc) {
  Header h;
  h.h0.x = 1u | ((uint32_t)format << 8) | ((uint32_t)flags << 16) | ((uint32_t)(dtype | (comp << 4)) << 24);
  h.h0.y = (uint32_t)d | ((uint32_t)n_vec << 16);
  h.h0.z = (uint32_t)(n_vec * d * 2);
  h.h0.w = stored;
  h.h1.x = (uint32_t)spill;
  h.h1.y = (uint32_t)(spill >> 32);
  h.h1.z = crc;
  h.h1.w = aux;
  return h;
}
__device__ __forceinline__ void write_desc(kvc_segment_desc* desc, uint64_t slot_off, int format, int flags,
                                           int status, int d, int n_vec, uint32_t stored, uint64_t spill,
                                           uint32_t crc) {
  uint4 d0, d1;
  d0.x = (uint32_t)slot_off;
  d0.y = (uint32_t)(slot_off >> 32);
  d0.z = (uint32_t)spill;
  d0.w = (uint32_t)(spill >> 32);
  d1.x = stored;
  d1.y = (uint32_t)(n_vec * d * 2);
  d1.z = 1u | ((uint32_t)format << 8) | ((uint32_t)flags << 16) | ((uint32_t)status << 24);
  d1.w = crc;
  reinterpret_cast<uint4*>(desc)[0] = d0;
  reinterpret_cast<uint4*>(desc)[1] = d1;
}
__device__ __forceinline__ void write_header_desc(uint8_t* slot, kvc_segment_desc* desc, uint64_t slot_off,
                                                  int format, int flags, int status, int dtype, int comp,
                                                  int d, int n_vec, uint32_t stored, uint64_t spill,
                                                  uint32_t aux, uint32_t crc) {
  const Header h = make_header(format, flags, dtype, comp, d, n_vec, stored, spill, aux, crc);
  st_global16(slot, h.h0);
  st_global16(slot + 16, h.h1);
  write_desc(desc, slot_off, format, flags, status, d, n_vec, stored, spill, crc);
}

// codes + metadata bytes of a coded segment (block layout)
__device__ __forceinline__ uint32_t payload_bytes(int codec, int d, uint32_t n_vec) {
  int bits = 8, meta = 0;
  switch (codec) {
    case C_U3: case C_TQ3: bits = 3; break;
    case C_U4: case C_TQ4: bits = 4; break;
    default: break;
  }
  if (codec == C_FP8Y || codec == C_INT8 || codec == C_U3 || codec == C_U4) meta = 4;
  if (codec == C_TQ3 || codec == C_TQ4) meta = 2;
  return n_vec * (uint32_t)(bits * d / 8 + meta);
}
// stored bytes of a coded segment and where they start in the slot: the
// codes and metadata blocks after the header, or the record codec's rows
__device__ __forceinline__ uint32_t stored_offset(int codec) {
  return codec == C_I8R ? kRowsOffset : kHeaderBytes;
}
__device__ __forceinline__ uint32_t payload_bytes(int codec, int d, uint32_t n_vec, uint32_t heads,
                                                  uint32_t row_bytes) {
  if (codec == C_I8R) return n_vec / heads * row_bytes;
  return payload_bytes(codec, d, n_vec);
}

// ------------------------------------------------------------------ CRC-32
// CRC-32 of zlib over a byte range [OKV-SF "Ownership, storage and GDS":
// every stored segment carries a CRC32], computed by all lanes of the
// workgroup from the tables in CrcTables (see there for the lane schedule).
// The register is preset to 0xFFFFFFFF by complementing the first word and
// the result is complemented at the end.

// register after the four bytes of x (x = register ^ next little-endian word),
// from the nibble tables t[k][v] (eight lookups: the update is linear).  The
// byte offset 4v of nibble k is (x << 2 or x >> 2, shifted) & 0x3C; with
// BYTESEL the three upper bytes of x << 2 and x >> 2 are masked in one
// byte-select AND each.  BYTESEL measured faster in the encode kernels and
// slower in the decode kernels, so each direction passes its own choice.
template <bool BYTESEL>
__device__ __forceinline__ uint32_t crc_word(uint32_t x, const uint32_t (*t)[16]) {
  const uint32_t ev = x << 2, od = x >> 2;
  const uint8_t* b = reinterpret_cast<const uint8_t*>(t);
  auto at = [b](int k, uint32_t off) { return *reinterpret_cast<const uint32_t*>(b + 64 * k + off); };
  uint32_t a[8];
  a[0] = at(0, ev & 0x3Cu);
  a[1] = at(1, od & 0x3Cu);
  if constexpr (BYTESEL) {
    a[2] = at(2, and3c_byte<1>(ev));
    a[3] = at(3, and3c_byte<1>(od));
    a[4] = at(4, and3c_byte<2>(ev));
    a[5] = at(5, and3c_byte<2>(od));
    a[6] = at(6, and3c_byte<3>(ev));
    a[7] = at(7, and3c_byte<3>(od));
  } else {
#pragma unroll
    for (int k = 2; k < 8; k++) a[k] = at(k, (x >> (4 * k - 2)) & 0x3Cu);
  }
  return xor3(xor3(a[0], a[1], a[2]), xor3(a[3], a[4], a[5]), a[6] ^ a[7]);
}
// x^i * s_lane mod P for the lanes of an NT-thread workgroup, as 16-byte
// groups [i / 4][lane]
template <int NT>
__device__ __forceinline__ const uint4* crc_lane_powers(const Tables* tables) {
  if constexpr (NT == 64) return reinterpret_cast<const uint4*>(tables->crc.pw64);
  else if constexpr (NT == 128) return reinterpret_cast<const uint4*>(tables->crc.pw128);
  else return reinterpret_cast<const uint4*>(tables->crc.pw256);
}

// The CRC tables in LDS: a static allocation that only the kernels built
// with CRC reference, at an address the compiler knows, so table offsets
// fold into the LDS loads.
template <bool CRC>
__device__ __forceinline__ CrcLds* crc_tables_lds() {
  if constexpr (CRC) {
    __shared__ CrcLds s_crc_tables;
    return &s_crc_tables;
  } else {
    return nullptr;
  }
}

// log2 of a workgroup's wave count: its lane set in CrcTables::tj
template <int NT>
constexpr int crc_lane_set() {
  static_assert(NT == 64 || NT == 128 || NT == 256, "CRC lane sets cover 1, 2 or 4 waves");
  return NT == 64 ? 0 : (NT == 128 ? 1 : 2);
}

// Copy the tables for NT lanes into LDS (all threads of the workgroup; the
// caller synchronises before the first use).
template <int NT>
__device__ __forceinline__ void load_crc_tables(CrcLds* dst, const CrcTables* src) {
  constexpr uint32_t kT = sizeof(src->t) / 16, kTj = sizeof(src->tj[0]) / 16;
  static_assert(kT + kTj <= NT, "one 16-byte unit per thread");
  const uint32_t u = threadIdx.x;
  if (u < kT + kTj) {
    const uint4* from = u < kT ? reinterpret_cast<const uint4*>(src->t) + u
                               : reinterpret_cast<const uint4*>(src->tj[crc_lane_set<NT>()]) + (u - kT);
    reinterpret_cast<uint4*>(dst)[u] = ld_global16(from);
  }
}

// How crc32_lanes carries each lane's register over the units after its
// last one (NT - 1 - lane of them):
// - kCarryPowers: r * s_lane as the xor of the 32 powers x^i * s_lane
//   selected by r's bits (eight 16-byte loads per lane, in flight during the
//   loop), then an xor over the lanes; the encode kernels' form;
// - kCarryChain: the same product from s_lane alone, multiplied by x
//   between the 32 steps (one-wave decode, the entropy stage's decode);
// - kCarryTree: no per-lane carry; lanes are combined in pairs, log2(NT)
//   levels deep, level b multiplying the lower lane's register by
//   x^(128 * 2^b) from nibble tables in LDS (multi-wave decode).
enum { kCarryPowers = 0, kCarryChain = 1, kCarryTree = 2 };

// Levels of the pairwise lane combination an NT-lane workgroup uses:
// log2(NT), multipliers x^(128 * 2^b) for b < log2(NT)
template <int NT>
constexpr int crc_levels() { return NT == 64 ? 6 : (NT == 128 ? 7 : 8); }

// The lane carry of the decode kernels: the level tables (3.5-4 KiB) pay
// for themselves in multi-wave workgroups; a one-wave workgroup, whose slot
// may be a single KiB, measured faster with the chain and no extra tables
template <int NT>
constexpr int decode_crc_carry() { return NT > 64 ? kCarryTree : kCarryChain; }

// The level tables in LDS, for kernels built with CRC that combine lanes in
// a tree (as crc_tables_lds)
template <int NT, bool CRC>
__device__ __forceinline__ uint32_t (*crc_levels_lds())[8][16] {
  if constexpr (CRC && decode_crc_carry<NT>() == kCarryTree) {
    __shared__ uint32_t s_crc_levels[crc_levels<NT>()][8][16];
    return s_crc_levels;
  } else {
    return nullptr;
  }
}

// Copy the level tables into LDS: every thread issues its loads before its
// first store (the caller synchronises before the first use)
template <int NT>
__device__ __forceinline__ void load_crc_levels(uint32_t (*dst)[8][16], const CrcTables* src) {
  constexpr uint32_t kUnits = crc_levels<NT>() * sizeof(src->lv[0]) / 16;
  constexpr int R = (kUnits + NT - 1) / NT;
  const uint4* from = reinterpret_cast<const uint4*>(src->lv);
  uint4 w[R];
#pragma unroll
  for (int r = 0; r < R; r++)
    w[r] = threadIdx.x + r * NT < kUnits ? ld_global16(from + threadIdx.x + r * NT) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < R; r++)
    if (threadIdx.x + r * NT < kUnits) reinterpret_cast<uint4*>(dst)[threadIdx.x + r * NT] = w[r];
}

// CRC32 of n bytes; load(o) returns the 16 bytes at offset o of the range
// (o a multiple of 16).  When n is not a multiple of 16 the 16-byte unit
// holding the last bytes must be readable as a whole.  Called by all NT
// threads of the workgroup (with NT > 64 it synchronises them); every thread
// returns the CRC.  tables: the call's tables (the lanes' powers); lv: the
// level tables in LDS (kCarryTree only).  CARRY picks the lane carry (see
// above); ENC masks nibbles with byte-select ANDs (the encode kernels').
// Each form measured faster where it is used.
template <int NT, int CARRY, bool ENC = CARRY == kCarryPowers, class Load>
__device__ __forceinline__ uint32_t crc32_lanes(const Load& load, uint32_t n, const CrcLds* ct, const Tables* tables,
                                                const uint32_t (*lv)[8][16] = nullptr) {
  constexpr int NPW = CARRY == kCarryPowers ? 8 : (CARRY == kCarryChain ? 1 : 0);
  const uint32_t lane = threadIdx.x;
  const uint32_t units = n >> 4;
  // virtual zero units in front make the unit count a multiple of NT (a zero
  // register stays zero over zero bytes), so lane NT - 1 holds the last unit
  const uint32_t pad = (NT - (units & (NT - 1))) & (NT - 1);
  const uint32_t rounds = (units + pad) / NT;
  // x^i * s_lane (s_lane = x^(128 (NT - 1 - lane))), as [i / 4][lane][i % 4]
  uint4 pw[NPW > 0 ? NPW : 1];
  if constexpr (NPW > 0) {
    const uint4* pws = crc_lane_powers<NT>(tables) + lane;
#pragma unroll
    for (int g = 0; g < NPW; g++) pw[g] = ld_global16(pws + g * NT);
  }
  uint32_t r = 0;
  // each round's unit is loaded one round ahead.  Only round 0 holds
  // padding (q < 0): a zero unit, over which the register stays zero.  The
  // initial register 0xFFFFFFFF is the inverted first word of unit 0.  Every
  // round but the last ends in the jump tables, the last in the plain ones.
  // A wave whose lanes all hold padding in round 0 starts at round 1.
  const int32_t q0 = (int32_t)lane - (int32_t)pad;
  const uint32_t k0 = __builtin_amdgcn_readfirstlane(rounds && (int32_t)(lane | (kCrcLanes - 1)) < (int32_t)pad);
  uint4 w = make_uint4(0, 0, 0, 0);
  const int32_t qf = q0 + (int32_t)(k0 * NT);
  if (k0 < rounds && qf >= 0) w = load(16u * (uint32_t)qf);
  if (qf == 0) w.x = ~w.x;
  for (uint32_t k = k0; k + 1 < rounds; k++) {
    const uint4 wn = load(16u * (uint32_t)(q0 + (int32_t)((k + 1) * NT)));   // q0 + NT > 0
    r = crc_word<ENC>(r ^ w.x, ct->t);
    r = crc_word<ENC>(r ^ w.y, ct->t);
    r = crc_word<ENC>(r ^ w.z, ct->t);
    r = crc_word<ENC>(r ^ w.w, ct->tj);
    w = wn;
  }
  if (rounds > k0) {
    r = crc_word<ENC>(r ^ w.x, ct->t);
    r = crc_word<ENC>(r ^ w.y, ct->t);
    r = crc_word<ENC>(r ^ w.z, ct->t);
    r = crc_word<ENC>(r ^ w.w, ct->t);
  }
  if constexpr (CARRY == kCarryTree) {
    // after level b, lane j (a multiple of 2^(b+1)) holds the register of
    // lanes j .. j + 2^(b+1) - 1 carried to the end of the last one's unit:
    // lane j's level-(b-1) register times x^(128 * 2^b), xor lane j + 2^b's
#pragma unroll
    for (int b = 0; b < 6; b++) r = crc_word<false>(r, lv[b]) ^ __shfl_down(r, 1 << b, kCrcLanes);
    if constexpr (NT == kCrcLanes) {
      r = __builtin_amdgcn_readfirstlane(r);
    } else {
      // wave w's register (its lane 0), carried over the 64 units per round
      // of each later wave: times x^(128 * 64 * (NT / 64 - 1 - w))
      const uint32_t later = NT / kCrcLanes - 1 - lane / kCrcLanes;
      if (later & 1) r = crc_word<false>(r, lv[6]);
      if constexpr (NT > 2 * kCrcLanes)
        if (later & 2) r = crc_word<false>(r, lv[7]);
    }
  } else {
    // carry each register over the units after its last one (NT - 1 - lane):
    // r * s_lane, the xor of x^i * s_lane over the coefficients i set in r
    // (coefficient i is bit 31 - i)
    uint32_t c = 0;
    if constexpr (CARRY == kCarryPowers) {
#pragma unroll
      for (int g = 0; g < 8; g++) {
        c = xor_and(c, (uint32_t)((int32_t)(r << (4 * g)) >> 31), pw[g].x);
        c = xor_and(c, (uint32_t)((int32_t)(r << (4 * g + 1)) >> 31), pw[g].y);
        c = xor_and(c, (uint32_t)((int32_t)(r << (4 * g + 2)) >> 31), pw[g].z);
        c = xor_and(c, (uint32_t)((int32_t)(r << (4 * g + 3)) >> 31), pw[g].w);
      }
    } else {
      uint32_t v = pw[0].x;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        c = xor_and(c, (uint32_t)((int32_t)(r << i) >> 31), v);
        if (i < 31) v = xor_and(v >> 1, 0u - (v & 1u), 0xEDB88320u);   // v * x
      }
    }
    r = wave_xor(c);
  }
  if constexpr (NT > kCrcLanes) {                                // xor the waves' registers
    __shared__ uint32_t s_part[NT / kCrcLanes];
    if ((lane & (kCrcLanes - 1)) == 0) s_part[lane / kCrcLanes] = r;
    __syncthreads();
    r = 0;
#pragma unroll
    for (int v = 0; v < NT / kCrcLanes; v++) r ^= s_part[v];
    __syncthreads();                                             // s_part is reused by the next call
  }
  // the ragged end (n mod 16 bytes), the same in every lane: whole words
  // through the tables, the last bytes bit by bit
  if (!units) r = 0xFFFFFFFFu;
  const uint32_t tail = n & 15;
  if (tail) {
    const uint4 w = load(16u * units);
    if (tail >= 4) r = crc_word<ENC>(r ^ w.x, ct->t);
    if (tail >= 8) r = crc_word<ENC>(r ^ w.y, ct->t);
    if (tail >= 12) r = crc_word<ENC>(r ^ w.z, ct->t);
    const uint32_t q = tail >> 2;
    uint32_t last = q == 0 ? w.x : (q == 1 ? w.y : (q == 2 ? w.z : w.w));
    for (uint32_t b = 0; b < (tail & 3); b++, last >>= 8) {
      r ^= last & 0xFFu;
      for (int i = 0; i < 8; i++) r = (r >> 1) ^ (0xEDB88320u & (0u - (r & 1u)));
    }
  }
  return ~r;
}
// ranges in global memory and in the LDS slot image
struct GlobalBytes {
  const uint8_t* p;
  __device__ __forceinline__ uint4 operator()(uint32_t o) const { return ld_global16(p + o); }
};
struct LdsBytes {
  const uint8_t* p;
  __device__ __forceinline__ uint4 operator()(uint32_t o) const { return *reinterpret_cast<const uint4*>(p + o); }
};
// a range copied while its CRC is taken: each unit read from src is also
// stored at the same offset of dst (crc32_lanes reads every unit once).  The
// range must be a whole number of units: a ragged end is read as a whole
// unit, which would be stored too (raw segments hold n_vec * D * 2 bytes, a
// multiple of 64).  STREAM: nontemporal stores, for a destination whose
// lines the units cover whole
template <bool STREAM>
struct CopiedBytes {
  const uint8_t* src;
  uint8_t* dst;
  __device__ __forceinline__ uint4 operator()(uint32_t o) const {
    const uint4 w = ld_stream16(src + o);
    if constexpr (STREAM) st_stream16(dst + o, w);
    else st_global16(dst + o, w);
    return w;
  }
};

template <int D, int DT, int NT>
__device__ __forceinline__ int encode_codec(int codec, const SegCtx& s, const Lane& ln, float fixed,
                                            const LaneSigns<D>& ls, const CellEntry* cells, uint8_t* image) {
  switch (codec) {
    case C_FP8D: return encode_segment_vectors<D, DT, C_FP8D, NT>(s, ln, fixed, ls, cells, image);
    case C_FP8F: return encode_segment_vectors<D, DT, C_FP8F, NT>(s, ln, fixed, ls, cells, image);
    case C_FP8Y: return encode_segment_vectors<D, DT, C_FP8Y, NT>(s, ln, fixed, ls, cells, image);
    case C_INT8: return encode_segment_vectors<D, DT, C_INT8, NT>(s, ln, fixed, ls, cells, image);
    case C_U3: return encode_segment_vectors<D, DT, C_U3, NT>(s, ln, fixed, ls, cells, image);
    case C_U4: return encode_segment_vectors<D, DT, C_U4, NT>(s, ln, fixed, ls, cells, image);
    case C_TQ3: return encode_segment_vectors<D, DT, C_TQ3, NT>(s, ln, fixed, ls, cells, image);
    case C_TQ4: return encode_segment_vectors<D, DT, C_TQ4, NT>(s, ln, fixed, ls, cells, image);
    case C_I8R: return encode_segment_vectors<D, DT, C_I8R, NT>(s, ln, fixed, ls, cells, image);
    default: return 0;
  }
}

// CRC32 of bytes the workgroup has just written to global memory: the
// barrier orders every wave's stores before they are read back.  Called by
// all threads; every thread returns the CRC.
template <int NT>
__device__ __forceinline__ uint32_t crc32_written(const uint8_t* b, uint32_t n, const CrcLds* ct, const Tables* tables) {
  __syncthreads();
  return crc32_lanes<NT, kCarryPowers>(GlobalBytes{b}, n, ct, tables);
}

// ------------------------------------------------------------------ encode kernel
// D = 256 fits 71 VGPRs without spilling: seven waves per SIMD instead of
// six (1.2-1.5% faster); the others keep the compiler's choice
template <int D, int DT, int NT, bool CRC>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(D == 256 ? 7 : 1))) void encode_kernel(
    CallParams p) {
  __shared__ CellEntry s_cells[kCells];
  __shared__ unsigned long long s_spill;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_stage[];   // p.stage_bytes
  CrcLds* const ct = crc_tables_lds<CRC>();

  const uint32_t seg = p.seg_base + blockIdx.x;       // segments [seg_base, seg_base + grid)
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry E = side_entry(p, 2 * l + comp);
  const int codec = (int)E.codec;
  if (codec == C_ANS) return;                                   // the entropy stage's own kernel
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = page_id(p, pi);
  // guard: the side table and page list come from memory; never follow a
  // base pointer outside the caller's set or a page id outside the pool
  if ((uint64_t)(uintptr_t)E.base < p.base_lo || (uint64_t)(uintptr_t)E.base > p.base_hi || page < 0 ||
      (uint32_t)page >= p.num_blocks || slot_off + E.slot_bytes > p.slot_region) {
    if (threadIdx.x == 0) reinterpret_cast<uint4*>(p.desc + seg)[1] = make_uint4(0, 0, (uint32_t)KVC_SEG_GUARD << 24, 0);
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
  s.walk_dh = p.walk_dh;
  s.walk_step = p.walk_step;
  s.walk_wrap = p.walk_wrap;
  s.linear_iters = p.linear_iters;
  s.row_bytes = p.row_bytes;
  const uint32_t raw_bytes = (uint32_t)s.n_vec * D * 2;
  const uint32_t slot_bytes = E.slot_bytes;
  kvc_segment_desc* desc = p.desc + seg;

  // CRC32 of the stored bytes, by wave 0, read back from global memory after
  // all waves have written them (the barrier orders the workgroup's stores
  // before the loads) or from the LDS slot image
  constexpr bool crc = CRC;
  constexpr int crc_flag = CRC ? KVC_FLAG_CRC32 : 0;
  if constexpr (CRC) load_crc_tables<NT>(ct, &p.tables->crc);

  const Lane ln = lane_info<D>();
  // a page whose vectors follow each other (v at element v * D) is the raw
  // slot body byte for byte: with CRC32 it is copied by the CRC's own pass
  // (its carry from one power word: 32 held across the 16-byte units of a
  // whole page would spill)
  const bool contiguous = s.sh == (uint32_t)D && s.st == (uint32_t)s.heads * D;
  if (codec == C_RAW) {                                        // raw by policy
    uint32_t c = 0;
    if (crc && contiguous) {
      c = crc32_lanes<NT, kCarryChain, true>(
          CopiedBytes<false>{reinterpret_cast<const uint8_t*>(s.src), s.slot + kHeaderBytes}, raw_bytes, ct, p.tables);
    } else {
      copy_out_raw<D, NT, false>(s, ln, s.slot + kHeaderBytes);
      if (crc) c = crc32_written<NT>(s.slot + kHeaderBytes, raw_bytes, ct, p.tables);
    }
    zero_pad<NT>(s.slot, kHeaderBytes + raw_bytes, slot_bytes);
    if (threadIdx.x == 0)
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_POLICY | crc_flag, KVC_SEG_RAW_POLICY, DT,
                        comp, D, s.n_vec, raw_bytes, 0, 0, c);
    return;
  }

  const bool tq = codec == C_TQ3 || codec == C_TQ4;
  if (tq) {
    const uint2* src = reinterpret_cast<const uint2*>(p.tables->cells[codec == C_TQ4 ? 1 : 0]);
    uint2* dst = reinterpret_cast<uint2*>(s_cells);
    static_assert(sizeof(CellEntry) == sizeof(uint2), "one 8-byte word per cell");
    constexpr int R = (kCells + NT - 1) / NT;
    uint2 c[R];
#pragma unroll
    for (int r = 0; r < R; r++)
      c[r] = threadIdx.x + r * NT < kCells ? src[threadIdx.x + r * NT] : make_uint2(0, 0);
#pragma unroll
    for (int r = 0; r < R; r++)
      if (threadIdx.x + r * NT < kCells) dst[threadIdx.x + r * NT] = c[r];
    __syncthreads();
  }
  LaneSigns<D> ls;
  if (tq) make_lane_signs<D>(p.sign_mask, ln.p, true, ls);
  const float fixed = E.fixed;

  const uint32_t payload = payload_bytes(codec, D, (uint32_t)s.n_vec, p.heads, p.row_bytes);
  const uint32_t stored_at = stored_offset(codec);
  const bool rows = codec == C_I8R;

  // The slot body (codes, metadata, zero padding) is assembled in LDS when it
  // fits, then written with full-line nontemporal stores; partial-line
  // nontemporal stores straight from the lanes would not be merged.
  int bad;
  const bool staged = slot_bytes <= p.stage_bytes;
  if (staged) {
    bad = encode_codec<D, DT, NT>(codec, s, ln, fixed, ls, s_cells, s_stage);
    if (rows) zero_row_gaps<NT>(s_stage, p.tokens, p.heads, D, p.row_bytes, slot_bytes);
    else zero_pad<NT>(s_stage, kHeaderBytes + payload, slot_bytes);
  } else {
    bad = encode_codec<D, DT, NT>(codec, s, ln, fixed, ls, s_cells, s.slot);
    if (rows) zero_row_gaps<NT>(s.slot, p.tokens, p.heads, D, p.row_bytes, slot_bytes);
    else zero_pad<NT>(s.slot, kHeaderBytes + payload, slot_bytes);
  }
  const int any_bad = __syncthreads_or(bad);
  const uint32_t aux = codec == C_FP8F ? __float_as_uint(fixed) : 0u;
  if (staged && !any_bad) {
    const uint32_t c = crc ? crc32_lanes<NT, kCarryPowers>(LdsBytes{s_stage + stored_at}, payload, ct, p.tables) : 0u;
    // header + body from unit 0, so every wave store covers whole lines
    // the header goes into the image's first 32 bytes; the threads that
    // store them read them back below, in order after their own LDS stores
    if (threadIdx.x < 2) {
      const Header h = make_header(codec, crc_flag, DT, comp, D, s.n_vec, payload, 0, aux, c);
      if (threadIdx.x == 0) *reinterpret_cast<uint4*>(s_stage) = h.h0;
      if (threadIdx.x == 1) *reinterpret_cast<uint4*>(s_stage + 16) = h.h1;
    }
    for (uint32_t u = threadIdx.x; u < slot_bytes / 16; u += NT)
      st_stream16(s.slot + 16 * u, *reinterpret_cast<const uint4*>(s_stage + 16 * u));
    if (threadIdx.x == 0) write_desc(desc, slot_off, codec, crc_flag, KVC_SEG_ENCODED, D, s.n_vec, payload, 0, c);
    return;
  }
  // the slot body: the staged image of a coded segment; a segment raw
  // because of its data keeps only its header in the slot, and the rest of
  // the slot is zero.  Codes written straight to an unstaged slot before the
  // gate are overwritten: each wave first waits for its own stores to
  // complete, and a barrier orders them before the zeroing stores.
  if (any_bad && !staged) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (staged || any_bad)
    for (uint32_t u = 2 + threadIdx.x; u < slot_bytes / 16; u += NT)
      st_stream16(s.slot + 16 * u, any_bad ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(s_stage + 16 * u));
  if (!any_bad) {
    const uint32_t c = crc ? crc32_written<NT>(s.slot + stored_at, payload, ct, p.tables) : 0u;
    if (threadIdx.x == 0)
      write_header_desc(s.slot, desc, slot_off, codec, crc_flag, KVC_SEG_ENCODED, DT, comp, D, s.n_vec, payload, 0,
                        aux, c);
    return;
  }
  // raw because of its data: reserve spill space, copy the source bytes
  const uint64_t need = (raw_bytes + kSlotAlign - 1) / kSlotAlign * kSlotAlign;
  if (threadIdx.x == 0) s_spill = spill_reserve(p, need);
  __syncthreads();
  const uint64_t off = s_spill;
  const bool fits = p.slot_region + off + raw_bytes <= p.buf_bytes;
  // a segment that was not stored (no spill space) carries no CRC
  uint32_t c = 0;
  if (fits && crc && contiguous) {
    c = crc32_lanes<NT, kCarryChain, true>(
        CopiedBytes<true>{reinterpret_cast<const uint8_t*>(s.src), p.buf + p.slot_region + off}, raw_bytes, ct,
        p.tables);
  } else if (fits) {
    copy_out_raw<D, NT, true>(s, ln, p.buf + p.slot_region + off);
    if (crc) c = crc32_written<NT>(p.buf + p.slot_region + off, raw_bytes, ct, p.tables);
  }
  if (threadIdx.x == 0) {
    if (fits)
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_DATA | crc_flag, KVC_SEG_RAW_DATA, DT, comp,
                        D, s.n_vec, raw_bytes, p.slot_region + off, 0, c);
    else
      write_header_desc(s.slot, desc, slot_off, KVC_RAW, KVC_FLAG_RAW_DATA | KVC_FLAG_CAPACITY, KVC_SEG_CAPACITY,
                        DT, comp, D, s.n_vec, raw_bytes, 0, 0, 0);
  }
}

// ------------------------------------------------------------------ decoders
// the codes of one chunk (8 elements) of a vector's code block
template <int D, int BITS>
__device__ __forceinline__ uint2 load_codes(const uint8_t* slot, uint32_t cv, int k, int p) {
  constexpr int P = Geo<D>::P;
  const uint32_t e0 = k * 8 * P + 8 * p;
  if constexpr (BITS == 8) {
    return *byte_at(reinterpret_cast<const uint2*>(slot), cv + e0);
  } else if constexpr (BITS == 4) {
    return make_uint2(*byte_at(reinterpret_cast<const uint32_t*>(slot), cv + e0 / 2), 0u);
  } else {
    const uint8_t* q = byte_at(slot, cv + (3 * e0) / 8);
    return make_uint2((uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16), 0u);
  }
}

// byte m of a word, as a float (v_cvt_f32_ubyte*)
__device__ __forceinline__ float ubyte_f32(uint32_t w, int m) { return (float)((w >> (8 * m)) & 0xFFu); }

// what a lane reads of one stored vector: its code chunks and the metadata
template <int D>
struct VecCodes {
  uint2 c[Geo<D>::NCH];
  uint32_t meta;
};

// cv, mv: byte offsets of the vector's codes and metadata in the slot
template <int D, int C>
__device__ __forceinline__ void load_vec_codes(const uint8_t* slot, uint32_t cv, uint32_t mv, const Lane& ln,
                                               VecCodes<D>& vc) {
  constexpr int BITS = CodecInfo<C>::bits, META = CodecInfo<C>::meta;
#pragma unroll
  for (int k = 0; k < Geo<D>::NCH; k++) vc.c[k] = load_codes<D, BITS>(slot, cv, k, ln.p);
  if constexpr (META == 4) vc.meta = *byte_at(reinterpret_cast<const uint32_t*>(slot), mv);
  else if constexpr (META == 2) vc.meta = *byte_at(reinterpret_cast<const uint16_t*>(slot), mv);
  else vc.meta = 0;
}

template <int D, int DT, int C>
__device__ __forceinline__ void decode_vector(const VecCodes<D>& vc, const Lane& ln, uint16_t* page, uint32_t voff,
                                              float fixed,
                                              const LaneSigns<D>& ls, const float* cent) {
  constexpr int E = Geo<D>::E, NCH = Geo<D>::NCH, LOGP = Geo<D>::LOGP, P = Geo<D>::P;
  constexpr int BITS = CodecInfo<C>::bits;
  float y[E];
  if constexpr (CodecInfo<C>::fp8 || C == C_INT8 || C == C_I8R) {
    float s = 1.0f;
    if constexpr (C == C_FP8F) s = fixed;
    if constexpr (C == C_FP8Y || C == C_INT8) s = __uint_as_float(vc.meta);
    if constexpr (C == C_I8R) s = __uint_as_float(vc.meta << 16);          // BF16 scale
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const uint2 c = vc.c[k];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t word = j < 4 ? c.x : c.y;
        float val;
        if constexpr (C == C_INT8 || C == C_I8R) {
          val = (float)(int8_t)(word >> (8 * (j & 3)));
        } else {
          switch (j & 3) {
            case 0: val = __builtin_amdgcn_cvt_f32_fp8((int)word, 0); break;
            case 1: val = __builtin_amdgcn_cvt_f32_fp8((int)word, 1); break;
            case 2: val = __builtin_amdgcn_cvt_f32_fp8((int)word, 2); break;
            default: val = __builtin_amdgcn_cvt_f32_fp8((int)word, 3); break;
          }
        }
        if constexpr (C != C_FP8D) val = val * s;
        y[8 * k + j] = val;
      }
    }
  }
  if constexpr (CodecInfo<C>::uni) {
    const uint32_t mw = vc.meta;
    const float mh = (float)__builtin_bit_cast(_Float16, (uint16_t)(mw & 0xFFFFu));
    const float sh = (float)__builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const uint32_t w = vc.c[k].x;
      float code[8];
      if constexpr (BITS == 4) {
        const uint32_t even = w & 0x0F0F0F0Fu, odd = (w >> 4) & 0x0F0F0F0Fu;   // nibbles to bytes
#pragma unroll
        for (int m = 0; m < 4; m++) {
          code[2 * m] = ubyte_f32(even, m);
          code[2 * m + 1] = ubyte_f32(odd, m);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; j++) code[j] = (float)((w >> (BITS * j)) & ((1u << BITS) - 1));
      }
#pragma unroll
      for (int j = 0; j < 8; j++) y[8 * k + j] = fmaf(code[j], sh, mh);   // code*sh is exact
    }
  }
  if constexpr (CodecInfo<C>::tq) {
    // centroids, negated in lanes of odd group parity (cent + 16 holds -C)
    const int base = (__builtin_popcount(ln.p) & 1) ? 16 : 0;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const uint32_t w = vc.c[k].x;
#pragma unroll
      for (int j = 0; j < 8; j++) y[8 * k + j] = cent[base + ((w >> (BITS * j)) & ((1u << BITS) - 1))];
    }
    const float q = sumsq_tree<NCH, LOGP>(y);
    wht_inlane_low<NCH>(y);
    wht_cross<LOGP, E>(y, ln.p);
    wht_inlane_high<NCH>(y);
    const float nh = (float)__builtin_bit_cast(_Float16, (uint16_t)vc.meta);
    const float rd = sqrtf((float)D);
    const float g = nh / (sqrtf(q) * rd);
#pragma unroll
    for (int e = 0; e < E; e++) y[e] = y[e] * g;
  }
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    uint4 o = pack8<DT>(y + 8 * k);
    if constexpr (CodecInfo<C>::tq) {        // sigma_i on the packed output (sign bits 15, 31)
      o.x ^= ls.flip[4 * k];
      o.y ^= ls.flip[4 * k + 1];
      o.z ^= ls.flip[4 * k + 2];
      o.w ^= ls.flip[4 * k + 3];
    }
    st_global16(byte_at(page, 2 * (voff + 8 * ln.p) + 16 * P * k), o);
  }
}

// image: the slot's bytes -- staged in LDS, or the encoded buffer itself
template <int D, int DT, int C, int NT>
__device__ __forceinline__ void decode_segment_vectors(const SegCtx& s, const Lane& ln, float fixed,
                                                       const LaneSigns<D>& ls, const float* cent,
                                                       const uint8_t* image) {
  constexpr int GW = Geo<D, NT>::GW, U = Geo<D>::U;      // vectors whose codes are in flight together
  constexpr int CB = CodecInfo<C>::bits * D / 8;
  const uint32_t meta_blk = kHeaderBytes + (uint32_t)s.n_vec * CB;
  uint16_t* page = const_cast<uint16_t*>(s.src);
  if (s.linear_iters) {
    // vector v at element v * D, every batch full (see encode_segment_vectors)
#pragma unroll 1
    for (uint32_t it = 0; it < s.linear_iters; it++) {
      const int v0 = ln.g + (int)it * (GW * U);
      VecCodes<D> vc[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        uint32_t cv, mv;
        vec_offsets<D, C>(s, v0 + u * GW, meta_blk, cv, mv);
        load_vec_codes<D, C>(image, cv, mv, ln, vc[u]);
      }
#pragma unroll
      for (int u = 0; u < U; u++)      // (always true: keeps the vectors apart, as in encode)
        if (v0 + u * GW < s.n_vec) decode_vector<D, DT, C>(vc[u], ln, page, (uint32_t)(v0 + u * GW) * D, fixed, ls, cent);
    }
    return;
  }
  VecPos pos = vec_pos(s, ln.g);
  for (int v0 = ln.g; v0 < s.n_vec; v0 += GW * U) {
    VecCodes<D> vc[U];
#pragma unroll
    for (int u = 0; u < U; u++)
      if (v0 + u * GW < s.n_vec) {
        uint32_t cv, mv;
        vec_offsets<D, C>(s, v0 + u * GW, meta_blk, cv, mv);
        load_vec_codes<D, C>(image, cv, mv, ln, vc[u]);
      }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (v0 + u * GW < s.n_vec) decode_vector<D, DT, C>(vc[u], ln, page, pos.off, fixed, ls, cent);
      vec_advance(s, pos);
    }
  }
}

// copy a segment from contiguous canonical order into the engine layout
template <int D, int NT>
__device__ void copy_in_raw(const SegCtx& s, const Lane& ln, const uint8_t* srcb) {
  constexpr int P = Geo<D>::P, NCH = Geo<D>::NCH, GW = Geo<D, NT>::GW, U = Geo<D>::U;
  uint16_t* page = const_cast<uint16_t*>(s.src);
  VecPos pos = vec_pos(s, ln.g);
  for (int v0 = ln.g; v0 < s.n_vec; v0 += GW * U) {
    uint4 w[U][NCH];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int v = v0 + u * GW;
      if (v < s.n_vec) {
        const uint32_t b = (uint32_t)v * (2 * D) + 16 * ln.p;
#pragma unroll
        for (int k = 0; k < NCH; k++) w[u][k] = ld_global16(byte_at(srcb, b + 16 * P * k));
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (v0 + u * GW < s.n_vec) {
        const uint32_t b = 2 * (pos.off + 8 * ln.p);
#pragma unroll
        for (int k = 0; k < NCH; k++) st_global16(byte_at(page, b + 16 * P * k), w[u][k]);
      }
      vec_advance(s, pos);
    }
  }
}

template <int D, int DT, int NT>
__device__ __forceinline__ void decode_codec(int codec, const SegCtx& s, const Lane& ln, float fixed,
                                             const LaneSigns<D>& ls, const float* cent, const uint8_t* image) {
  switch (codec) {
    case C_FP8D: decode_segment_vectors<D, DT, C_FP8D, NT>(s, ln, fixed, ls, cent, image); break;
    case C_FP8F: decode_segment_vectors<D, DT, C_FP8F, NT>(s, ln, fixed, ls, cent, image); break;
    case C_FP8Y: decode_segment_vectors<D, DT, C_FP8Y, NT>(s, ln, fixed, ls, cent, image); break;
    case C_INT8: decode_segment_vectors<D, DT, C_INT8, NT>(s, ln, fixed, ls, cent, image); break;
    case C_U3: decode_segment_vectors<D, DT, C_U3, NT>(s, ln, fixed, ls, cent, image); break;
    case C_U4: decode_segment_vectors<D, DT, C_U4, NT>(s, ln, fixed, ls, cent, image); break;
    case C_TQ3: decode_segment_vectors<D, DT, C_TQ3, NT>(s, ln, fixed, ls, cent, image); break;
    case C_TQ4: decode_segment_vectors<D, DT, C_TQ4, NT>(s, ln, fixed, ls, cent, image); break;
    case C_I8R: decode_segment_vectors<D, DT, C_I8R, NT>(s, ln, fixed, ls, cent, image); break;
    default: break;
  }
}

// D <= 128 fits 64 VGPRs without spilling: eight waves per SIMD instead of
// seven, more slots and pages in flight per CU (the CRC and one-wave decodes
// measured 1.5-3.6% faster); at D = 256 that bound would spill
template <int D, int DT, int NT, bool CRC>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 8 : 1))) void decode_kernel(
    CallParams p) {
  __shared__ float s_cent[32];
  extern __shared__ __attribute__((aligned(16))) uint8_t s_stage[];   // p.stage_bytes
  CrcLds* const ct = crc_tables_lds<CRC>();
  uint32_t (*const lvs)[8][16] = crc_levels_lds<NT, CRC>();
  const uint32_t seg = p.seg_base + blockIdx.x;       // segments [seg_base, seg_base + grid)
  const uint32_t two_n = 2u * p.n_pages;
  const uint32_t l = seg / two_n;
  const uint32_t rem = seg - l * two_n;
  const uint32_t pi = rem >> 1, comp = rem & 1;
  const SideEntry E = side_entry(p, 2 * l + comp);
  const int codec = (int)E.codec;
  if (codec == C_ANS) return;                                   // the entropy stage's own kernel
  const uint64_t slot_off = E.slot_base + (uint64_t)pi * E.page_stride;
  const int32_t page = page_id(p, pi);
  if ((uint64_t)(uintptr_t)E.base < p.base_lo || (uint64_t)(uintptr_t)E.base > p.base_hi || page < 0 ||
      (uint32_t)page >= p.num_blocks || slot_off + E.slot_bytes > p.slot_region) {
    if (p.seg_status && threadIdx.x == 0) p.seg_status[seg] = 2;
    return;
  }
  SegCtx s;
  s.src = E.base + (int64_t)page * p.sb;                  // destination page
  s.slot = p.buf + slot_off;
  s.heads = (int)p.heads;
  s.heads_magic = p.heads_magic;
  s.n_vec = (int)(p.heads * p.tokens);
  s.st = p.st32;
  s.sh = p.sh32;
  s.walk_dh = p.walk_dh;
  s.walk_step = p.walk_step;
  s.walk_wrap = p.walk_wrap;
  s.linear_iters = p.linear_iters;
  s.row_bytes = p.row_bytes;
  const uint32_t raw_bytes = (uint32_t)s.n_vec * D * 2;

  // A coded slot that fits is read whole into LDS with 16-byte loads (header
  // and codes together); otherwise the header is read first.
  const uint32_t slot_bytes = E.slot_bytes;
  const bool staged = codec != C_RAW && slot_bytes <= p.stage_bytes;
  if constexpr (CRC) {
    load_crc_tables<NT>(ct, &p.tables->crc);
    if constexpr (decode_crc_carry<NT>() == kCarryTree) load_crc_levels<NT>(lvs, &p.tables->crc);
  }
  // TurboQuant centroids (negated in s_cent[16..31]) and the lane's signs.
  // A one-wave workgroup, whose life is mostly memory latency, issues their
  // loads with the slot's; larger ones load them once the slot is in LDS
  // (measured faster there).
  const bool tq = codec == C_TQ3 || codec == C_TQ4;
  constexpr bool early = NT == 64;
  const Lane ln = lane_info<D>();
  float cent = 0.0f;
  LaneSigns<D> ls;
  if (early && tq) {
    if (threadIdx.x < 32) cent = p.tables->centroids[codec == C_TQ4 ? 1 : 0][threadIdx.x & 15];
    make_lane_signs<D>(p.sign_mask, ln.p, false, ls);
  }
  uint4 h0, h1;
  if (staged) {
    // kStageRounds units per thread are loaded before any is stored to LDS,
    // so a wave waits for one memory latency per kStageRounds units, not one
    // per unit
    const uint32_t nu = slot_bytes / 16;
    for (uint32_t u0 = threadIdx.x; u0 < nu; u0 += kStageRounds * NT) {
      uint4 w[kStageRounds];
#pragma unroll
      for (int r = 0; r < kStageRounds; r++)
        if (u0 + r * NT < nu) w[r] = ld_stream16(s.slot + 16 * (u0 + r * NT));
#pragma unroll
      for (int r = 0; r < kStageRounds; r++)
        if (u0 + r * NT < nu) *reinterpret_cast<uint4*>(s_stage + 16 * (u0 + r * NT)) = w[r];
    }
    if (early && tq && threadIdx.x < 32) s_cent[threadIdx.x] = threadIdx.x < 16 ? cent : -cent;
    __syncthreads();                                      // the slot image (and the centroids)
    h0 = *reinterpret_cast<const uint4*>(s_stage);
    h1 = *reinterpret_cast<const uint4*>(s_stage + 16);
  } else {
    if (early && tq && threadIdx.x < 32) s_cent[threadIdx.x] = threadIdx.x < 16 ? cent : -cent;
    h0 = ld_global16(s.slot);
    h1 = ld_global16(s.slot + 16);
  }
  const int version = h0.x & 0xFF, format = (h0.x >> 8) & 0xFF, flags = (h0.x >> 16) & 0xFF;
  const int dc = (h0.x >> 24) & 0xFF;
  bool ok = version == 1 && dc == (DT | (int)(comp << 4)) && (h0.y & 0xFFFF) == (uint32_t)D &&
            (h0.y >> 16) == (uint32_t)s.n_vec && h0.z == raw_bytes;
  const bool raw_data = flags & KVC_FLAG_RAW_DATA;
  uint64_t spill = (uint64_t)h1.x | ((uint64_t)h1.y << 32);
  if (raw_data) ok = ok && format == KVC_RAW && !(flags & KVC_FLAG_CAPACITY) && raw_bytes <= p.buf_bytes &&
                     spill >= p.slot_region && spill <= p.buf_bytes - raw_bytes;
  else ok = ok && format == codec;
  const uint32_t stored =
      raw_data || codec == C_RAW ? raw_bytes : payload_bytes(codec, D, (uint32_t)s.n_vec, p.heads, p.row_bytes);
  const uint32_t stored_at = stored_offset(codec);
  ok = ok && h0.w == stored && ((flags & KVC_FLAG_CRC32) != 0) == CRC;
  if (!ok) {
    if (p.seg_status && threadIdx.x == 0) p.seg_status[seg] = 1;
    return;
  }
  // the stored bytes must match the header's CRC32 before the page is written
  if constexpr (CRC) {
    __syncthreads();                                      // CRC tables in LDS
    const uint32_t c =
        raw_data ? crc32_lanes<NT, decode_crc_carry<NT>()>(GlobalBytes{p.buf + spill}, stored, ct, p.tables, lvs)
        : staged ? crc32_lanes<NT, decode_crc_carry<NT>()>(LdsBytes{s_stage + stored_at}, stored, ct, p.tables, lvs)
                 : crc32_lanes<NT, decode_crc_carry<NT>()>(GlobalBytes{s.slot + stored_at}, stored, ct, p.tables, lvs);
    if (c != h1.z) {
      if (p.seg_status && threadIdx.x == 0) p.seg_status[seg] = 3;
      return;
    }
  }
  if (p.seg_status && threadIdx.x == 0) p.seg_status[seg] = 0;

  if (raw_data || codec == C_RAW) {
    const uint8_t* from = raw_data ? p.buf + spill : s.slot + kHeaderBytes;
    // four-wave workgroups copy a page stored in canonical order flat (one
    // round of loads instead of two; 1% faster on the benchmark decode, and
    // measured slower for one-wave workgroups and in encode)
    if (NT > 64 && s.sh == (uint32_t)D && s.st == (uint32_t)s.heads * D)
      copy_flat<NT>(from, reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(s.src)), raw_bytes);
    else copy_in_raw<D, NT>(s, ln, from);
    return;
  }
  if (!early && tq) {
    if (threadIdx.x < 32) {
      const float c = p.tables->centroids[codec == C_TQ4 ? 1 : 0][threadIdx.x & 15];
      s_cent[threadIdx.x] = threadIdx.x < 16 ? c : -c;
    }
    make_lane_signs<D>(p.sign_mask, ln.p, false, ls);
  }
  if (tq && (!early || !staged)) __syncthreads();         // the centroids
  const float fixed = __uint_as_float(h1.w);
  if (staged) decode_codec<D, DT, NT>(codec, s, ln, fixed, ls, s_cent, s_stage);
  else decode_codec<D, DT, NT>(codec, s, ln, fixed, ls, s_cent, s.slot);
}

// ------------------------------------------------------------------ entropy stage
#include "kvc_ans_device.h"

// ------------------------------------------------------------------ allocation-free scratch
// The scratch of kvc_encode_pages_noalloc, one copy per GPU for the life of
// the process.  In host code `scratch` names a host-side stand-in, never the
// device array: only the address from hipGetSymbolAddress is used.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// dynamic LDS of a launch: the slot staging
inline uint32_t dynamic_lds(const CallParams& p) { return p.stage_bytes; }

template <int D, int DT, int NT, bool CRC>
struct EncodeLaunch {
  static void run(const CallParams& p, uint64_t n, hipStream_t st) {
    hipLaunchKernelGGL((encode_kernel<D, DT, NT, CRC>), dim3((unsigned)n), dim3(NT), dynamic_lds(p), st, p);
  }
};
template <int D, int DT, int NT, bool CRC>
struct DecodeLaunch {
  static void run(const CallParams& p, uint64_t n, hipStream_t st) {
    hipLaunchKernelGGL((decode_kernel<D, DT, NT, CRC>), dim3((unsigned)n), dim3(NT), dynamic_lds(p), st, p);
  }
};
// instantiation for the call's dtype, workgroup size (one wave, or BIG
// threads; BIGC with the CRC option) and CRC option; a launch with another
// size is refused
template <int D, int BIG, int BIGC, template <int, int, int, bool> class F>
hipError_t dispatch(const CallParams& p, uint64_t nseg, hipStream_t st) {
  const bool bf = p.dtype == KVC_BF16, small = p.threads == kThreadsSmall, crc = p.crc != 0;
  if (!small && p.threads != (uint32_t)(crc ? BIGC : BIG)) return hipErrorInvalidConfiguration;
  if (bf) {
    if (small) crc ? F<D, KVC_BF16, kThreadsSmall, true>::run(p, nseg, st) : F<D, KVC_BF16, kThreadsSmall, false>::run(p, nseg, st);
    else crc ? F<D, KVC_BF16, BIGC, true>::run(p, nseg, st) : F<D, KVC_BF16, BIG, false>::run(p, nseg, st);
  } else {
    if (small) crc ? F<D, KVC_FP16, kThreadsSmall, true>::run(p, nseg, st) : F<D, KVC_FP16, kThreadsSmall, false>::run(p, nseg, st);
    else crc ? F<D, KVC_FP16, BIGC, true>::run(p, nseg, st) : F<D, KVC_FP16, BIG, false>::run(p, nseg, st);
  }
  return hipGetLastError();
}
template <int D>
hipError_t launch_encode_d(const CallParams& p, uint64_t nseg, hipStream_t st) {
  return dispatch<D, kEncodeThreads, kEncodeThreadsCrc, EncodeLaunch>(p, nseg, st);
}
template <int D>
hipError_t launch_decode_d(const CallParams& p, uint64_t nseg, hipStream_t st) {
  return dispatch<D, kDecodeThreads, kDecodeThreads, DecodeLaunch>(p, nseg, st);
}

}  // namespace

hipError_t noalloc_scratch(int device, const Tables* host_tables, uint8_t** ptr) {
  static std::mutex mu;
  static uint8_t* addr[kNoAllocMaxDevices] = {};
  if (device < 0 || device >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    e = hipMemcpy(p, host_tables, sizeof(Tables), hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    addr[device] = static_cast<uint8_t*>(p);
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_encode(const CallParams& p, uint32_t head_dim, uint64_t nseg, hipStream_t st) {
  switch (head_dim) {
    case 32: return launch_encode_d<32>(p, nseg, st);
    case 64: return launch_encode_d<64>(p, nseg, st);
    case 128: return launch_encode_d<128>(p, nseg, st);
    case 256: return launch_encode_d<256>(p, nseg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ans_encode(const CallParams& p, uint32_t head_dim, uint64_t nseg, hipStream_t st) {
  const bool crc = p.crc != 0;
  switch (head_dim) {
    case 32: crc ? launch_ans_encode_dc<32, true>(p, nseg, st) : launch_ans_encode_dc<32, false>(p, nseg, st); break;
    case 64: crc ? launch_ans_encode_dc<64, true>(p, nseg, st) : launch_ans_encode_dc<64, false>(p, nseg, st); break;
    case 128: crc ? launch_ans_encode_dc<128, true>(p, nseg, st) : launch_ans_encode_dc<128, false>(p, nseg, st); break;
    case 256: crc ? launch_ans_encode_dc<256, true>(p, nseg, st) : launch_ans_encode_dc<256, false>(p, nseg, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ans_decode(const CallParams& p, uint32_t head_dim, uint64_t nseg, hipStream_t st) {
  const bool crc = p.crc != 0;
  switch (head_dim) {
    case 32: crc ? launch_ans_decode_dc<32, true>(p, nseg, st) : launch_ans_decode_dc<32, false>(p, nseg, st); break;
    case 64: crc ? launch_ans_decode_dc<64, true>(p, nseg, st) : launch_ans_decode_dc<64, false>(p, nseg, st); break;
    case 128: crc ? launch_ans_decode_dc<128, true>(p, nseg, st) : launch_ans_decode_dc<128, false>(p, nseg, st); break;
    case 256: crc ? launch_ans_decode_dc<256, true>(p, nseg, st) : launch_ans_decode_dc<256, false>(p, nseg, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const CallParams& p, uint32_t head_dim, uint64_t nseg, hipStream_t st) {
  switch (head_dim) {
    case 32: return launch_decode_d<32>(p, nseg, st);
    case 64: return launch_decode_d<64>(p, nseg, st);
    case 128: return launch_decode_d<128>(p, nseg, st);
    case 256: return launch_decode_d<256>(p, nseg, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvc
