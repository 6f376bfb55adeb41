// Chunk-parallel half of the chunkwise WY/UT prefill (gfx950): the fused form of the prep
// kernel (chunk_prep_impl.h), one workgroup per (batch, value head, chunk), for every gate
// layout and input prologue.
#include "chunk_prep_impl.h"

namespace gdr {

hipError_t launch_prep_fused(const LaunchArgs& a) { return dispatch_prep_form<false>(a); }

}  // namespace gdr
