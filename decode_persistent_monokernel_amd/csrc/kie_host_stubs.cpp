// Host-only stand-ins for the device-side helpers that the HIP sources
// define, for the sanitizer build of the host library (kie_api.cpp compiled
// with the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer).
// That build runs the CPU tests of the C ABI: argument checks, sizes, the
// packer and the schedule validator.  It never launches anything; every
// helper reports that no device code is present.
#include <hip/hip_runtime_api.h>

#include "kie_layout.h"

extern "C" hipError_t kie_internal_launch_ring8(const kie::KParams*, int, size_t, hipStream_t) {
  return hipErrorNoBinaryForGpu;
}
extern "C" hipError_t kie_internal_launch_ring10(const kie::KParams*, int, size_t, hipStream_t) {
  return hipErrorNoBinaryForGpu;
}
extern "C" hipError_t kie_internal_zero_ring8(void*, size_t, hipStream_t) { return hipErrorNoBinaryForGpu; }
extern "C" hipError_t kie_internal_occupancy_ring8(int, int, size_t, int*) { return hipErrorNoBinaryForGpu; }
extern "C" hipError_t kie_internal_occupancy_ring10(int, int, size_t, int*) { return hipErrorNoBinaryForGpu; }
extern "C" hipError_t kie_internal_prefill_chunk(const kie::PrefillArgs*, hipStream_t) {
  return hipErrorNoBinaryForGpu;
}
extern "C" hipError_t kie_internal_noalloc_scratch(int, void**) { return hipErrorNoBinaryForGpu; }
