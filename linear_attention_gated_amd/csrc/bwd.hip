// bwd.hip -- backward kernels (in progress).
#include "frag.h"
#include "gdn_internal.h"

namespace gdn {
hipError_t launch_bwd_prep(const Params&, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_state(const Params&, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_grad(const Params&, int, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdn
