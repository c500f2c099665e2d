// gdn2_wide.h -- exact in-chunk decay factors for chunks whose decay spans a
// wide range, shared by the chunk-parallel kernels.
//
// The chunkwise WY form (arXiv 2605.22791 abstract; research-wiki summary,
// "Key findings") needs the decay between two tokens of a chunk,
// exp(g_r - g_i) <= 1 for i <= r (g the in-chunk cumulative log-decay of one
// channel), inside the Gram matrices A = strict_lower((b k) k^T) and
// P = lower_incl(q k^T) and inside the backward's products with them. The
// fast path factors it through the chunk middle m, exp(g_r - g_m) exp(g_m - g_i),
// which is exact only while |g - g_m| stays inside fp32's exponent range.
// A chunk where some channel's |g_r - g_m| exceeds kWideSpan takes the wide
// path instead, where no factor ever exceeds 1:
//
//   gb_r   cumulative log-decay from the start of r's 16-token block (rows
//          16R .. r), so differences of it never cancel large values;
//   Bs_R   the total of block R;
//   tiles of 16-token blocks R > I:
//     exp(g_r - g_i) = exp(gb_r) * exp(sum_{I<J<R} Bs_J) * exp(Bs_I - gb_i),
//     three factors <= 1: the row factor, a per-channel pair scale (1 when
//     I = R - 1) and the column factor; the products run on fp32 matrix cores;
//   diagonal blocks (R = I): exp(gb_r - gb_i) for every pair, in fp32 VALU.
//
// Every per-token log-decay is floored at kLaFloor inside the chunked
// kernels, so a single token never decays a channel by more than
// exp(-20) ~ 2.1e-9 there (below fp32's relative resolution of 6e-8 next to
// any term of order one); this keeps the cumulative sums finite (log-decay
// -inf is a valid input: a channel reset) and bounds them, which bounds their
// rounding. The one-token decode kernel applies exp(log_alpha) exactly.
#pragma once

#include "gdn2_common.h"

namespace gdn2 {

constexpr float kLaFloor = -20.f;
constexpr float kWideSpan = 60.f;
// workgroups of a wide-chunk pass: one per compute unit (the pass's LDS admits one workgroup per
// CU, so more would only queue); each reads the flags of about items / kWideGrid chunks, kWideBatch
// at a time, in parallel
constexpr int kWideGrid = 256;
constexpr int kWideBatch = 64;
// the single-pass forward's mark of a sequence that met a wide chunk: a quiet NaN with a payload that
// no arithmetic produces (an input NaN carrying it only makes the sequence recompute, exactly)
constexpr uint32_t kWideMark = 0x7fc0d1deu;

// NaN stays NaN (an fmaxf would replace it)
__device__ __forceinline__ float la_floor(float x) { return x < kLaFloor ? kLaFloor : x; }

// block pairs (R, I) with I <= R - 2 carry a pair scale; their index
__host__ __device__ constexpr int wide_npair(int NB) { return NB > 2 ? (NB - 1) * (NB - 2) / 2 : 0; }
__device__ __forceinline__ int wide_pair(int R, int I) { return (R - 2) * (R - 1) / 2 + I; }
__device__ __forceinline__ void wide_pair_rc(int p, int& R, int& I) {
  R = 2;
  while (p > R - 2) {
    p -= R - 1;
    ++R;
  }
  I = p;
}

// Per-channel block tables from the block totals Bs [NB][DK] (fp32 LDS):
// pair scales sPS[wide_pair(R, I)][c] = exp(sum_{I<J<R} Bs[J][c]). All threads
// of the workgroup call it; the caller synchronises before and after.
template <int NB, int DK, int NT>
__device__ __forceinline__ void wide_pair_scales(const float* sBs, float* sPS) {
  for (int e = threadIdx.x; e < wide_npair(NB) * DK; e += NT) {
    const int p = e / DK, c = e - p * DK;
    int R, I;
    wide_pair_rc(p, R, I);
    float s = 0.f;
    for (int J = I + 1; J < R; ++J) s += sBs[J * DK + c];
    sPS[e] = __expf(s);
  }
}

// Sum of the block totals before / after block R of channel c.
template <int NB, int DK>
__device__ __forceinline__ float wide_before(const float* sBs, int R, int c) {
  float s = 0.f;
#pragma unroll
  for (int J = 0; J < NB; ++J) s += J < R ? sBs[J * DK + c] : 0.f;
  return s;
}
template <int NB, int DK>
__device__ __forceinline__ float wide_after(const float* sBs, int R, int c) {
  float s = 0.f;
#pragma unroll
  for (int J = NB - 1; J >= 0; --J) s += J > R ? sBs[J * DK + c] : 0.f;
  return s;
}

// C += (X diag(s)) Y^T on fp32 matrix cores, X and Y fp32 in LDS K-contiguous
// ([16][K] rows at ldx / ldy); s (per contraction index) may be null.
template <int K>
__device__ __forceinline__ void mma_nt_f32s(f32x4& acc, const float* X, int ldx, const float* Y, int ldy,
                                            const float* s) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) {
    float x = X[r * ldx + k0 + g];
    if (s) x *= s[k0 + g];
    acc = mfma16x16x4(x, Y[r * ldy + k0 + g], acc);
  }
}

// Exact diagonal 16x16 blocks of the decay-weighted Gram matrices for one
// channel slice:
//   A_ri += sum_c bk_rc k_ic exp(gb_rc - gb_ic)    (i < r, same 16-token block)
//   P_ri += sum_c q_rc  k_ic exp(gb_rc - gb_ic)    (i <= r)
// The calling thread owns row r and the 4 channels cs..cs+3 of the slice (TPR
// consecutive lanes share a row); sK and sGb hold k and gb of every row of the
// slice (fp32, row stride ld). The row sums over the TPR lanes go to
// tA / tP [rows][16] at column i - 16 * (r / 16). Every lane of the wave must
// call it (the row sums are wave shuffles); rows with !live contribute zeros
// and rows >= C write nothing.
template <int TPR, int C>
__device__ __forceinline__ void gram_diag_pairwise(int r, bool live, int cs, const float (&bk)[4],
                                                   const float (&q)[4], const float (&gb)[4], const float* sK,
                                                   const float* sGb, int ld, float* tA, float* tP) {
  float pa[16], pp[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pa[i] = pp[i] = 0.f;
  const int R0 = r & ~15, rl = r & 15;
  if (live) {
#pragma unroll
    for (int il = 0; il < 16; ++il) {
      if (il <= rl) {
        const float4 k4 = *reinterpret_cast<const float4*>(sK + (R0 + il) * ld + cs);
        const float4 g4 = *reinterpret_cast<const float4*>(sGb + (R0 + il) * ld + cs);
        const float kk[4] = {k4.x, k4.y, k4.z, k4.w}, gg[4] = {g4.x, g4.y, g4.z, g4.w};
        float ta = 0.f, tp = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float t = kk[j] * __expf(gb[j] - gg[j]);
          ta += bk[j] * t;
          tp += q[j] * t;
        }
        pa[il] = il < rl ? ta : 0.f;
        pp[il] = tp;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < TPR; m *= 2) {
#pragma unroll
    for (int il = 0; il < 16; ++il) {
      pa[il] += __shfl_xor(pa[il], m, kWave);
      pp[il] += __shfl_xor(pp[il], m, kWave);
    }
  }
  const int c4 = lane_id() % TPR;
  if (r < C) {
#pragma unroll
    for (int il = 0; il < 16; ++il) {
      if ((il * TPR) / 16 == c4) {
        tA[r * 16 + il] = pa[il];
        tP[r * 16 + il] = pp[il];
      }
    }
  }
}

}  // namespace gdn2
