// gdn2_bwd_d64.hip -- per-chunk gradient kernels for d_k = 64 (gdn2_bwd_impl.h).

#include "gdn2_bwd_impl.h"

namespace gdn2 {

hipError_t launch_grad_d64(const BwdArgs& a, hipStream_t s) {
  return a.f32_inputs ? launch_grad_dk<64, true>(a, s) : launch_grad_dk<64, false>(a, s);
}

}  // namespace gdn2
