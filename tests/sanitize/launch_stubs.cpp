// launch_stubs.cpp -- stand-ins for the kernel launchers, for the host-only
// sanitizer build of the C ABI (the driver never gets past validation; if a
// call did, these abort so that the run fails).
#include <cstdio>
#include <cstdlib>

#include "../../linear_attention_gated_amd/csrc/gdn_internal.h"

extern "C" const char* abi_driver_case(void);   // the driver's current case

namespace gdn {
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "a launch was reached in the host-only build: %s (case: %s)\n", what, abi_driver_case());
  std::abort();
}
hipError_t launch_plan(const Params&, hipStream_t) { reached("plan"); }
hipError_t launch_fwd_prep(const Params&, int, bool, hipStream_t) { reached("fwd_prep"); }
hipError_t launch_fwd_state(const Params&, int, bool, bool, hipStream_t) { reached("fwd_state"); }
hipError_t launch_fwd_out(const Params&, int, bool, hipStream_t) { reached("fwd_out"); }
hipError_t launch_bwd_prep(const Params&, int, bool, hipStream_t) { reached("bwd_prep"); }
hipError_t launch_bwd_state(const Params&, int, bool, hipStream_t) { reached("bwd_state"); }
hipError_t launch_bwd_grad(const Params&, int, bool, hipStream_t) { reached("bwd_grad"); }
int gnorm_blocks(long long rows, int, bool, bool) { return rows > 0 ? 1 : 0; }
hipError_t launch_gnorm_fwd(const GnormParams&, int, bool, hipStream_t) { reached("gnorm_fwd"); }
hipError_t launch_gnorm_bwd(const GnormParams&, int, bool, hipStream_t) { reached("gnorm_bwd"); }
hipError_t launch_gnorm_dw(const GnormParams&, int, bool, hipStream_t) { reached("gnorm_dw"); }
int conv_bwd_rows(long long tokens, int) { return tokens > 0 ? 1 : 0; }
hipError_t launch_conv_fwd(const ConvParams&, bool, hipStream_t) { reached("conv_fwd"); }
hipError_t launch_conv_bwd(const ConvParams&, bool, hipStream_t) { reached("conv_bwd"); }
hipError_t launch_conv_dw(const ConvParams&, hipStream_t) { reached("conv_dw"); }
hipError_t launch_recurrent(const RecParams&, int, int, bool, hipStream_t) { reached("recurrent"); }
}  // namespace gdn
