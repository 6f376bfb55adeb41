// Stand-ins for the kernel launchers of libgdr, so that the host entry points (gdr_api.cpp)
// can be built alone with host sanitizers and driven without a GPU: every launch reports
// that no device is present, as the HIP runtime does on a machine without one.
#include "gdr_launch.h"

namespace gdr {

hipError_t launch_tokens(const LaunchArgs&) { return hipErrorNoDevice; }
hipError_t launch_prep_fused(const LaunchArgs&) { return hipErrorNoDevice; }
hipError_t launch_prep_split(const LaunchArgs&) { return hipErrorNoDevice; }
hipError_t launch_chunk_carry(const LaunchArgs&) { return hipErrorNoDevice; }
hipError_t launch_carry_split(const LaunchArgs&) { return hipErrorNoDevice; }
hipError_t launch_tree_verify(const LaunchArgs&, const int32_t*) { return hipErrorNoDevice; }
hipError_t launch_varlen_plan(const LaunchArgs&) { return hipErrorNoDevice; }

}  // namespace gdr
