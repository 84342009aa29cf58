// Backward of multi-head differential attention (placeholder until the fused
// kernels land): reports that the configuration is not available.
#include "common.h"
#include "kernels.h"

namespace diffattn {

size_t bwd_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_bwd(const BwdParams &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace diffattn
