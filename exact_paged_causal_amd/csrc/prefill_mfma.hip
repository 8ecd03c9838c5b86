// prefill_mfma.hip -- tiled causal prefill on the matrix cores (placeholder
// until the tiled kernel lands: reports "not supported" so the C ABI returns
// ATLAS_ERR_UNSUPPORTED instead of running anything else).
#include "kernels.h"

namespace atlas {

hipError_t launch_prefill_mfma(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace atlas
