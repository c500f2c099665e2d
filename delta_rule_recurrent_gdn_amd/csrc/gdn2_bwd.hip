// gdn2_bwd.hip -- gate-aware chunkwise backward (placeholder until the kernels land).
#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
bool bwd_supported(int, int, int, bool) { return false; }

}  // namespace gdn2
