// gdn2_bwd.hip -- dispatch of the per-chunk gradient pass of the chunkwise backward
// (kernels in gdn2_bwd_impl.h, compiled per key width in gdn2_bwd_d*.hip so that
// the instantiations build in parallel).

#include "gdn2_bwd_impl.h"

namespace gdn2 {

hipError_t launch_grad_d16(const BwdArgs& a, hipStream_t s);
hipError_t launch_grad_d32(const BwdArgs& a, hipStream_t s);
hipError_t launch_grad_d64(const BwdArgs& a, hipStream_t s);
hipError_t launch_grad_d128(const BwdArgs& a, hipStream_t s);
hipError_t launch_grad_d128_f32(const BwdArgs& a, hipStream_t s);

hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream) {
  switch (a.Dk) {
    case 16: return launch_grad_d16(a, stream);
    case 32: return launch_grad_d32(a, stream);
    case 64: return launch_grad_d64(a, stream);
    case 128: return a.f32_inputs ? launch_grad_d128_f32(a, stream) : launch_grad_d128(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int DK, bool F32IN>
static bool grad_fits_c(int chunk) {
  switch (chunk) {
    case 16: return GradCfg<DK, 16, F32IN>::kFits;
    case 32: return GradCfg<DK, 32, F32IN>::kFits;
    case 64: return GradCfg<DK, 64, F32IN>::kFits;
  }
  return false;
}

bool grad_supported(int Dk, int chunk, bool f32) {
  switch (Dk) {
    case 16: return f32 ? grad_fits_c<16, true>(chunk) : grad_fits_c<16, false>(chunk);
    case 32: return f32 ? grad_fits_c<32, true>(chunk) : grad_fits_c<32, false>(chunk);
    case 64: return f32 ? grad_fits_c<64, true>(chunk) : grad_fits_c<64, false>(chunk);
    case 128: return f32 ? grad_fits_c<128, true>(chunk) : grad_fits_c<128, false>(chunk);
  }
  return false;
}

}  // namespace gdn2
