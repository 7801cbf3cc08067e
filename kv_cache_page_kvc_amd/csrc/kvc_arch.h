// kvc_arch.h -- gfx950-specific helpers of libkvc's kernels: global-memory
// access through address-space-1 pointers (global_load/global_store rather
// than flat, which would also count against the LDS wait counter), the
// DPP-fused FMA used by the cross-lane WHT butterflies, and short correctly
// rounded reciprocal and square-root sequences built on the hardware
// estimates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) uint32_t g_u32;

// 16-byte load of source pages, which are read once per call
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const g_u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_global16(const void* p) {
  const u32x4 v = *(const g_u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_global4(const void* p) { return *(const g_u32*)p; }
__device__ __forceinline__ uint2 ld_global8(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *(const __attribute__((address_space(1))) u32x2*)p;
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_global8(void* p, uint2 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 w = {v.x, v.y};
  *(__attribute__((address_space(1))) u32x2*)p = w;
}
__device__ __forceinline__ void st_global16(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  *(g_u32x4*)p = w;
}

// Nontemporal 16-byte store, for encoded slots written whole lines at a time
// (on gfx950 that raises the write rate of the encode stream; stores of
// partial lines are not merged and must not use it).
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (g_u32x4*)p);
}

// x as a binary32 register value: an empty asm the compiler cannot look
// through, so a later rounding of x (to FP16, say) is not merged into the
// instruction that produced x (e.g. an FMA fused with the FP16 conversion,
// which would round once instead of twice).
__device__ __forceinline__ float materialize_f32(float x) {
  asm("" : "+v"(x));
  return x;
}

// y[e] += c * y[e] of the partner lane, for e < 8, in one v_fmac_f32_dpp
// each (single rounding; c = +-1 makes the product exact).  Partner of
// stage Q: lane xor 1 (Q=0), xor 2 (Q=1), xor 8 within the row (Q=2), xor 7
// within the half-row (Q=3, row_half_mirror).
// The compiler does not see DPP inside the asm, so the block opens with
// five wait states (a VALU write of a VGPR needs two before a DPP read of
// it, a VALU write of EXEC five) and closes with two, for any DPP reader
// of its results that the compiler places right after it.
#define KVC_FMAC_DPP8(CTRL)                                                                        \
  asm("s_nop 4\n\t"                                                                                \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
      "s_nop 1"                                                                                    \
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7]) \
      : "v"(c))

// Group minimum and maximum over the lanes of a vector group: partners lane
// xor 1, xor 2 (LOGP >= 2), xor 8 (LOGP >= 3) and xor 7 (LOGP == 4), each
// step one v_min_f32_dpp / v_max_f32_dpp with the partner lane.  The hardware min/max is used directly (no
// quieting of signalling NaNs): callers detect NaN separately.  Two wait
// states separate each step from the previous one (DPP reads of a VGPR
// written by VALU), five open the block.
#define KVC_MINMAX_STEP(CTRL)                                                                      \
  "v_min_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                             \
  "v_max_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                             \
  "s_nop 1\n\t"
template <int LOGP>
__device__ __forceinline__ void group_minmax_dpp(float& mn, float& mx) {
  if constexpr (LOGP == 1)
    asm("s_nop 4\n\t" KVC_MINMAX_STEP("quad_perm:[1,0,3,2]") : "+v"(mn), "+v"(mx));
  else if constexpr (LOGP == 2)
    asm("s_nop 4\n\t" KVC_MINMAX_STEP("quad_perm:[1,0,3,2]") KVC_MINMAX_STEP("quad_perm:[2,3,0,1]")
        : "+v"(mn), "+v"(mx));
  else if constexpr (LOGP == 3)
    asm("s_nop 4\n\t" KVC_MINMAX_STEP("quad_perm:[1,0,3,2]") KVC_MINMAX_STEP("quad_perm:[2,3,0,1]")
            KVC_MINMAX_STEP("row_ror:8")
        : "+v"(mn), "+v"(mx));
  else
    asm("s_nop 4\n\t" KVC_MINMAX_STEP("quad_perm:[1,0,3,2]") KVC_MINMAX_STEP("quad_perm:[2,3,0,1]")
            KVC_MINMAX_STEP("row_ror:8") KVC_MINMAX_STEP("row_half_mirror")
        : "+v"(mn), "+v"(mx));
}
#undef KVC_MINMAX_STEP

// Bitwise helpers the compiler does not form by itself around LDS results:
// byte B of x masked with 0x3C as one v_and_b32 with a byte-select source
// operand, a ^ b ^ c and a ^ (b & c) as one v_bitop3_b32 each.
template <int B>
__device__ __forceinline__ uint32_t and3c_byte(uint32_t x) {
  static_assert(B >= 1 && B <= 3, "byte 1, 2 or 3 (byte 0 is a plain AND)");
  uint32_t r;
  if constexpr (B == 1)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(0x3Cu), "v"(x));
  else if constexpr (B == 2)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(0x3Cu), "v"(x));
  else
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(0x3Cu), "v"(x));
  return r;
}
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t xor_and(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x78" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// RN(1/h) by one Newton step e = 1 - h*y0, y0 + e*y0 from the hardware
// estimate y0 (accurate to one ulp), for
//  - every positive finite h that is an FP16 value: every start within one
//    ulp of 1/h gives the correctly rounded reciprocal (checked exhaustively
//    on the CPU), so the estimate's own rounding does not matter;
//  - every binary32 h in [2^-48, 2^16): the same holds for every start but
//    one per binade (h = (2 - 2^-23) * 2^k started at 2^-(k+1), a fixed point
//    of the step, as of every longer Newton sequence), and the device's own
//    estimate followed by the step equals the IEEE quotient for every such h
//    (checked exhaustively on the device).
__device__ __forceinline__ float recip_newton(float h) {
  const float y0 = __builtin_amdgcn_rcpf(h);
  return fmaf(fmaf(-h, y0, 1.0f), y0, y0);
}

// Correctly rounded square root of a binary32 S in [2^-96, 2^31), without
// the range scaling and special-value handling of the general sequence: the
// hardware estimate s (accurate to one ulp) gives way to its lower or upper
// neighbour s' when the sign of the residual S - s'*s shows the root past
// the midpoint between them.  In that range a nonzero residual is at least
// 2^-144 in magnitude, so its sign survives the FMA's rounding.  Exact for
// every start within one ulp of the root (checked exhaustively on the CPU).
__device__ __forceinline__ float sqrt_rn_normal(float S) {
  const float s = __builtin_amdgcn_sqrtf(S);
  const float sd = __uint_as_float(__float_as_uint(s) - 1u), su = __uint_as_float(__float_as_uint(s) + 1u);
  const float t = fmaf(-sd, s, S) <= 0.0f ? sd : s;
  return fmaf(-su, s, S) > 0.0f ? su : t;
}

template <int Q>
__device__ __forceinline__ void fmac_xlane8(float* y, float c) {
  if constexpr (Q == 0) KVC_FMAC_DPP8("quad_perm:[1,0,3,2]");
  else if constexpr (Q == 1) KVC_FMAC_DPP8("quad_perm:[2,3,0,1]");
  else if constexpr (Q == 2) KVC_FMAC_DPP8("row_ror:8");
  else KVC_FMAC_DPP8("row_half_mirror");
}

#undef KVC_FMAC_DPP8

}  // namespace kvc
