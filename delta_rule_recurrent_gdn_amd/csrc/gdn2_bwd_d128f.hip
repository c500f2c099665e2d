// gdn2_bwd_d128f.hip -- per-chunk gradient kernels for d_k = 128, fp32 inputs (gdn2_bwd_impl.h).

#include "gdn2_bwd_impl.h"

namespace gdn2 {

hipError_t launch_grad_d128_f32(const BwdArgs& a, hipStream_t s) { return launch_grad_dk<128, true>(a, s); }

}  // namespace gdn2
