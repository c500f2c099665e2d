// gdn2_gscale.hip -- partial maxima of the upstream gradients for the 16-bit
// backward's power-of-two prescale (grad_scale() in gdn2_internal.h).
//
// The gate-aware backward (arXiv 2605.22791 abstract) is linear in (dO,
// dS_final) jointly; its matrix-core operands for them are fp16, whose normal
// range (6.1e-5 .. 65504) is far narrower than that of the bf16 inputs. One
// workgroup per ((sequence, head), split) reads a kGradScaleSplit-th of the
// sequence's dO rows (and of its dS_final rows) and writes max |x| to
// part[state * kGradScaleSplit + split]; the backward kernels combine the
// partial maxima themselves, so nothing needs clearing between calls.

#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

__global__ __launch_bounds__(256) void gdn2_grad_scale_kernel(BwdArgs a, float* part) {
  const int st = blockIdx.x / kGradScaleSplit, sp = blockIdx.x - st * kGradScaleSplit;
  const SeqLoc sl = seq_loc(a.vl, a.T, a.H, a.Dk, a.Dv, a.chunk, st);
  const int t_lo = (int)((int64_t)sl.len * sp / kGradScaleSplit);
  const int t_hi = (int)((int64_t)sl.len * (sp + 1) / kGradScaleSplit);
  const int64_t rowV = (int64_t)a.H * a.Dv;
  const int g8 = a.Dv / 8;  // 16-byte groups per row
  const uint16_t* dO = static_cast<const uint16_t*>(a.dO);
  float m = 0.f;
  for (int e = threadIdx.x; e < (t_hi - t_lo) * g8; e += 256) {
    const int t = t_lo + e / g8, j = e - (e / g8) * g8;
    const uint4 u = *reinterpret_cast<const uint4*>(dO + sl.baseV + (int64_t)(sl.tok0 + t) * rowV + 8 * j);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
    }
  }
  if (a.dS_final) {
    const int r_lo = a.Dk * sp / kGradScaleSplit, r_hi = a.Dk * (sp + 1) / kGradScaleSplit;
    const float* S = a.dS_final + (int64_t)st * a.Dk * a.Dv;
    for (int e = r_lo * a.Dv + threadIdx.x; e < r_hi * a.Dv; e += 256) m = fmaxf(m, fabsf(S[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    part[(int64_t)st * kGradScaleSplit + sp] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

hipError_t launch_grad_scale(const BwdArgs& a, float* part, hipStream_t s) {
  const int nst = seq_items(a.vl, a.B, a.H);
  if (nst <= 0) return hipSuccess;
  hipLaunchKernelGGL(gdn2_grad_scale_kernel, dim3((unsigned)nst * kGradScaleSplit), dim3(256), 0, s, a, part);
  return hipGetLastError();
}

}  // namespace gdn2
