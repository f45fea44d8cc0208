// Host-only stand-ins for the kernel launchers (test infrastructure): the API
// layer (csrc/rmsq_api.cpp) is built with the host compiler under the
// address and undefined-behaviour sanitizers and linked with these, so its
// argument validation, shape choice and aliasing checks run on the CPU.  A
// call that passes every check reaches one of these and fails as a launch.
#include "rmsq_internal.h"

namespace rmsq {

namespace {
hipError_t no_device() { return hipErrorNoDevice; }
}  // namespace

hipError_t launch_fp8_gated(const FusedArgs&, const void*, const void*, int, bool, Shape, hipStream_t) {
    return no_device();
}
hipError_t launch_fp8(const FusedArgs&, int, bool, int, Shape, hipStream_t) { return no_device(); }
hipError_t launch_fp8_phased(const FusedArgs&, int, bool, int, Shape, hipStream_t) { return no_device(); }
hipError_t launch_fp8_elem(const FusedArgs&, int, bool, int, Shape, hipStream_t) { return no_device(); }
hipError_t launch_fp8_sum(const SumArgs&, int, int, Shape, hipStream_t) { return no_device(); }
hipError_t launch_fp4(const FusedArgs&, int, bool, Fp4Format, Shape, hipStream_t) { return no_device(); }
hipError_t launch_convert(int, const void*, void*, int64_t, hipStream_t) { return no_device(); }
hipError_t launch_wide(const FusedArgs&, int, bool, int, Fp4Format, int, hipStream_t) { return no_device(); }

}  // namespace rmsq
