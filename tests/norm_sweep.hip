// norm_sweep.hip -- test-only kernel: the TurboQuant encoder's short
// correctly rounded sequences (kvc_arch.h: sqrt_rn_normal on [2^-96, 2^31),
// recip_newton on [2^-48, 2^16)) evaluated on the device for every binary32
// input of a range and compared with the IEEE double-precision result
// rounded to binary32 (no square root or reciprocal of a binary32 value lies
// within 2^-49 of a binary32 midpoint, so that double rounding is exact).
// Not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_arch.h"

namespace {

// inputs first .. first + count - 1 (bit patterns); which = 0: square root,
// 1: reciprocal.  Adds the number of mismatches to *bad and lowers
// *first_bad to the smallest mismatching pattern.
__global__ __launch_bounds__(256) void norm_sweep(uint32_t first, uint32_t count, int which,
                                                  unsigned long long* bad, uint32_t* first_bad) {
  const uint32_t stride = gridDim.x * 256u;
  unsigned long long nbad = 0;
  uint32_t fb = 0xFFFFFFFFu;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < count; i += stride) {
    const uint32_t b = first + i;
    const float x = __uint_as_float(b);
    float got, ref;
    if (which == 0) {
      got = kvc::sqrt_rn_normal(x);
      ref = (float)__dsqrt_rn((double)x);
    } else {
      got = kvc::recip_newton(x);
      ref = (float)__ddiv_rn(1.0, (double)x);
    }
    if (__float_as_uint(got) != __float_as_uint(ref)) {
      nbad++;
      fb = min(fb, b);
    }
  }
  if (nbad) {
    atomicAdd(bad, nbad);
    atomicMin(first_bad, fb);
  }
}

}  // namespace

// Launch on `stream` (a hipStream_t, may be null).  count < 2^31; bad and
// first_bad are device words the caller has set (0 and 0xFFFFFFFF).
// Returns the launch status (hipSuccess = 0).
extern "C" int kvc_test_norm_sweep(uint32_t first, uint32_t count, int which, unsigned long long* bad,
                                   uint32_t* first_bad, void* stream) {
  if (count == 0) return 0;
  if (count >= 0x80000000u || (which != 0 && which != 1)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_sweep, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first, count, which,
                     bad, first_bad);
  return (int)hipGetLastError();
}
