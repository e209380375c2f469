// Launchers that launch nothing, for a host-only build of the C ABI's argument
// checks (kda_api.cpp and kda_sizes.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every one reports a HIP error, so a call that
// passes validation returns KDA_ERROR_HIP here instead of touching a device.
#include "kda_launch.h"

namespace kda {

hipError_t launch_recurrent_step(const StepArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_chunk_fwd(const ChunkArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_order_buffer(hipStream_t, int **out) {
    *out = nullptr;
    return hipErrorNoDevice;
}
hipError_t launch_order_sequences(const int *, int, int *, hipStream_t) { return hipErrorNoDevice; }
int plan_chunk_dvt(int, int, bool) { return 16; }
hipError_t launch_gdn2_step(const Gdn2StepArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gdn2_chunk_fwd(const Gdn2ChunkArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_backward(const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_chunk(const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }

}  // namespace kda
