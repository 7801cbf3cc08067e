// sanitize_stubs.cpp -- test infrastructure: stands in for the kernel
// launchers when the host half of libkvc (kvc_host.cpp) is built alone with
// AddressSanitizer and UndefinedBehaviorSanitizer for CPU tests of its
// argument validation and slot plan.  Nothing here is ever launched: every
// launcher reports that the device path is absent.
#include "kvc_internal.h"

namespace kvc {
hipError_t launch_encode(const CallParams&, uint32_t, uint64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const CallParams&, uint32_t, uint64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ans_encode(const CallParams&, uint32_t, uint64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ans_decode(const CallParams&, uint32_t, uint64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(int, const Tables*, uint8_t**) { return hipErrorNotSupported; }
}  // namespace kvc
