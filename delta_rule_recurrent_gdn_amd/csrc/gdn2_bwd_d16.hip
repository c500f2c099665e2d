// gdn2_bwd_d16.hip -- per-chunk gradient kernels for d_k = 16 (gdn2_bwd_impl.h).

#include "gdn2_bwd_impl.h"

namespace gdn2 {

hipError_t launch_grad_d16(const BwdArgs& a, hipStream_t s) {
  return a.f32_inputs ? launch_grad_dk<16, true>(a, s) : launch_grad_dk<16, false>(a, s);
}

}  // namespace gdn2
