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

// max |x| over a 16-byte group of bf16 values, on the magnitude bits (for values >= 0 the order of
// the bit patterns is that of the values)
__device__ __forceinline__ uint32_t absmax_bits(uint32_t m, const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return m;
}

constexpr int kScaleThreads = 256;
constexpr int kScaleUnroll = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kScaleThreads) void gdn2_grad_scale_kernel(BwdArgs a, float* part) {
  // heads fastest: the workgroups in flight read whole token rows (all heads' slices of a row) rather
  // than one head's 2*Dv-byte slice of rows H*Dv*2 bytes apart
  const int h = blockIdx.x % a.H, r = blockIdx.x / a.H;
  const int sq = r / kGradScaleSplit, sp = r - sq * kGradScaleSplit;
  const int st = sq * a.H + h;
  const SeqLoc sl = seq_loc(a.vl, a.T, a.H, a.Dk, a.Dv, a.chunk, st);
  const int t_lo = (int)((int64_t)sl.len * sp / kGradScaleSplit);
  const int t_hi = (int)((int64_t)sl.len * (sp + 1) / kGradScaleSplit);
  const int64_t rowV = (int64_t)a.H * a.Dv;
  const int g8 = a.Dv / 8, sh = __builtin_ctz(g8);  // 16-byte groups per row (Dv is a power of two)
  const int n = (t_hi - t_lo) * g8;
  const char* base = static_cast<const char*>(a.dO) + 2 * (sl.baseV + (int64_t)(sl.tok0 + t_lo) * rowV);
  uint32_t mb = 0;
  for (int e0 = threadIdx.x; e0 < n; e0 += kScaleThreads * kScaleUnroll) {
    uint4 u[kScaleUnroll];
#pragma unroll
    for (int i = 0; i < kScaleUnroll; ++i) {
      const int e = e0 + i * kScaleThreads, t = e >> sh, j = e & (g8 - 1);
      u[i] = e < n ? *reinterpret_cast<const uint4*>(base + 2 * ((int64_t)t * rowV + 8 * j))
                   : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kScaleUnroll; ++i) mb = absmax_bits(mb, u[i]);
  }
  float m = __uint_as_float(mb << 16);
  if (a.dS_final) {
    const int r_lo = a.Dk * sp / kGradScaleSplit, r_hi = a.Dk * (sp + 1) / kGradScaleSplit;
    const float4* S = reinterpret_cast<const float4*>(a.dS_final + (int64_t)st * a.Dk * a.Dv);
    for (int e = r_lo * a.Dv / 4 + threadIdx.x; e < r_hi * a.Dv / 4; e += kScaleThreads) {
      const float4 x = S[e];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  __shared__ float red[kScaleThreads / kWave];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kScaleThreads / kWave; ++i) r = fmaxf(r, red[i]);
    part[(int64_t)st * kGradScaleSplit + sp] = r;
  }
}

hipError_t launch_grad_scale(const BwdArgs& a, float* part, hipStream_t s) {
  const int nst = seq_items(a.vl, a.B, a.H);
  if (nst <= 0) return hipSuccess;
  hipLaunchKernelGGL(gdn2_grad_scale_kernel, dim3((unsigned)nst * kGradScaleSplit), dim3(kScaleThreads), 0, s, a, part);
  return hipGetLastError();
}

}  // namespace gdn2
