// Backward kernels (recompute form): placeholder until the gfx950 kernel lands.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace sap {

hipError_t launch_attn_bwd(const BwdLaunch &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace sap
