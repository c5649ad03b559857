// fa_bwd.hip -- backward pass (not yet implemented: reports unsupported).
#include "fa_internal.hpp"

namespace fa {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
