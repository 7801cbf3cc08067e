// fp8_cvt_sweep.hip -- test-only kernel: the gfx950 hardware E4M3FN
// conversion (v_cvt_pk_fp8_f32, round to nearest even, the instruction the
// encode kernels use for every FP8 code) applied to a range of binary32 bit
// patterns, so that a test can compare every pattern in [-448, 448] with the
// CPU oracle.  Not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// codes of patterns first + 4i .. first + 4i + 3 (modulo 2^32), packed
// little-endian into out[i], for i < groups
__global__ __launch_bounds__(256) void cvt_sweep(uint32_t first, uint32_t groups, uint32_t* out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= groups) return;
  const uint32_t b = first + 4u * i;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b), __uint_as_float(b + 1u), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b + 2u), __uint_as_float(b + 3u), w, true);
  out[i] = (uint32_t)w;
}

}  // namespace

// Launch on `stream` (a hipStream_t, may be null); out holds `groups`
// 32-bit words.  Returns the launch status (hipSuccess = 0).
extern "C" int kvc_test_fp8_cvt_sweep(uint32_t first, uint32_t groups, uint32_t* out, void* stream) {
  if (groups == 0) return 0;
  hipLaunchKernelGGL(cvt_sweep, dim3((groups + 255u) / 256u), dim3(256), 0, static_cast<hipStream_t>(stream), first,
                     groups, out);
  return (int)hipGetLastError();
}
