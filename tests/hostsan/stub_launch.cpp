// stub_launch.cpp -- the kernel launchers of fa_internal.hpp (and the
// static-scratch lookup) replaced by stubs that touch no device, so that the C-ABI layer (fa_api.cpp) and the
// host grid arithmetic (fa_host.cpp) can be built for the host alone, with
// AddressSanitizer and UndefinedBehaviorSanitizer, and driven by the ABI
// tests on a machine without a GPU. A call that passes validation reaches a
// stub, which reports an error: the ABI tests expect validation to stop
// every call they make before that point.
#include "fa_internal.hpp"

namespace fa {

hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipErrorInvalidDeviceFunction; }
hipError_t launch_fwd_fp8(const FwdArgs&, hipStream_t) { return hipErrorInvalidDeviceFunction; }
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorInvalidDeviceFunction; }
hipError_t static_scratch(void**) { return hipErrorNoDevice; }

}  // namespace fa
