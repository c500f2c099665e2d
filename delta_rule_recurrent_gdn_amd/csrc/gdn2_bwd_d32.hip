// gdn2_bwd_d32.hip -- per-chunk gradient kernels for d_k = 32 (gdn2_bwd_impl.h).

#include "gdn2_bwd_impl.h"

namespace gdn2 {

hipError_t launch_grad_d32(const BwdArgs& a, hipStream_t s) {
  return a.f32_inputs ? launch_grad_dk<32, true>(a, s) : launch_grad_dk<32, false>(a, s);
}

}  // namespace gdn2
