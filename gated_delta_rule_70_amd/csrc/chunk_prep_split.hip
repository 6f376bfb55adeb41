// Chunk-parallel half of the chunkwise WY/UT prefill (gfx950): the split form of the prep
// kernel (chunk_prep_impl.h) for a gate shared per key head -- one workgroup per
// (batch, key head, chunk) computes the gram, causal terms and decayed operands once and
// solves per value head.
#include "chunk_prep_impl.h"

namespace gdr {

hipError_t launch_prep_split(const LaunchArgs& a) {
    if (a.HG != a.HK || a.HV / a.HK > kSplitMaxGroup) return hipErrorInvalidValue;
    return dispatch_prep_form<true>(a);
}

}  // namespace gdr
