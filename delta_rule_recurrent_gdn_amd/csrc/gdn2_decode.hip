// gdn2_decode.hip -- one-token decode step of the Gated Delta Rule-2 operator.
//
// Constant-memory decoding (arXiv 2605.22791 abstract): per (batch, head) the
// fp32 state S (Dk x Dv) is read once and written once:
//   S~ = Diag(alpha) S,  r = S~^T (b*k),  p = S~^T q,  u = w*v - r,
//   o  = p + (k.q) u,    S <- S~ + k u^T
// (o = S_new^T q expanded so that a single pass over S~ gives both reads).
//
// Roofline: HBM-bound. Per (b, h): 2 * 4 * Dk * Dv state bytes plus the small
// per-token vectors; about 7 flops per state element on the fp32 vector ALUs.
//
// Layout of the work: one workgroup per (b, h). Each thread owns 4 adjacent
// value columns (one float4) of RPT key rows; consecutive threads cover a row
// from left to right, so each wave-wide load or store touches one contiguous
// block of the state. Column partial sums of r and p are reduced across row
// groups through LDS.

#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <int DK, int DV>
struct DecodeShape {
  static constexpr int kCols4 = DV / 4;                               // threads per state row
  static constexpr int kThreads = (kCols4 * DK < 256) ? kCols4 * DK : 256;
  static constexpr int kRowGroups = kThreads / kCols4;
  static constexpr int kRowsPerThread = DK / kRowGroups;
  static_assert(kRowsPerThread >= 1 && kRowGroups * kRowsPerThread == DK, "decode tiling");
  static_assert((kRowsPerThread & (kRowsPerThread - 1)) == 0, "rows per thread: a power of two");
};

template <int DK, int DV, bool F32IN>
__global__ __launch_bounds__((DecodeShape<DK, DV>::kThreads)) void gdn2_decode_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int NT = Sh::kThreads, RG = Sh::kRowGroups, RPT = Sh::kRowsPerThread, C4 = Sh::kCols4;
  constexpr int NWAVES = (NT + kWave - 1) / kWave;

  __shared__ float s_alpha[DK], s_e[DK], s_q[DK], s_k[DK];
  __shared__ float s_red_r[RG][DV + 4], s_red_p[RG][DV + 4];
  __shared__ float s_wsum[NWAVES];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t vec_k = bh * DK, vec_v = bh * DV;
  // state: [B, H] in place, or entry b's slot of a state pool [num_slots, H]
  int64_t sidx = bh;
  if (a.slots) {
    const int bi = (int)(bh / a.H), h = (int)(bh - (int64_t)bi * a.H);
    const int slot = a.slots[bi];
    if (slot < 0 || slot >= a.num_slots) {  // no state for this entry: o = 0, nothing else
      for (int j = tid; j < DV; j += NT) a.o[vec_v + j] = 0.f;
      return;
    }
    sidx = (int64_t)slot * a.H + h;
  }
  float* S = a.S + sidx * (int64_t)DK * DV;

  // stream the state rows owned by this thread, first, so that their latency and
  // that of the per-channel vectors below overlap (the vectors' LDS writes wait
  // for every load issued before them); through a buffer resource over this
  // head's state: one VGPR offset and a scalar row offset per access
  const int j4 = tid % C4, rg = tid / C4;
  const __amdgpu_buffer_rsrc_t Sr = __builtin_amdgcn_make_buffer_rsrc(S, 0, DK * DV * 4, kBufferRsrcWord3);
  const int voff = (rg * DV + 4 * j4) * 4;
  constexpr int kRowStep = RG * DV * 4;  // bytes between a thread's rows
  // slot i holds the thread's row step (i + rot) mod RPT: neighbouring workgroups
  // start at different 4 KiB pieces of their states, which all begin on 64 KiB
  // boundaries (the same offsets at the same time otherwise)
  const int rot = (int)(blockIdx.x & (RPT - 1));
  auto row_of = [&](int i) { return (i + rot) & (RPT - 1); };
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(Sr, voff, row_of(i) * kRowStep, 0));
  // this thread's 4 value columns of v and w, in flight with the state
  float vv[4], wg[4];
  load4<F32IN>(a.v, vec_v + 4 * j4, vv);
  load4_gate<F32IN>(a.w, vec_v + 4 * j4, bh, a.scalar_w, wg);
  __builtin_amdgcn_sched_barrier(0);

  // per-channel key-side vectors
  float kq = 0.f;
  if (tid < DK) {
    const float qv = load1<F32IN>(a.q, vec_k + tid);
    const float kv = load1<F32IN>(a.k, vec_k + tid);
    // per-head scalar gates ([B, H]): one value for every channel
    float bv = load1<F32IN>(a.b, a.scalar_b ? bh : vec_k + tid);
    const float la = a.log_alpha[a.scalar_decay ? bh : vec_k + tid];
    // pre-activation gates: b = sigmoid(b_raw), alpha = exp(-softplus(a_raw)) = sigmoid(-a_raw)
    if (a.raw_gates) bv = sigmoid_f(bv);
    s_alpha[tid] = a.raw_gates ? sigmoid_f(-la) : expf(la);
    s_e[tid] = bv * kv;
    s_q[tid] = qv;
    s_k[tid] = kv;
    kq = kv * qv;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
  if ((tid & (kWave - 1)) == 0) s_wsum[tid / kWave] = kq;

  __syncthreads();

  float4 r = make_float4(0.f, 0.f, 0.f, 0.f), p = r;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * row_of(i);
    const float al = s_alpha[c], e = s_e[c], qc = s_q[c];
    s[i].x *= al; s[i].y *= al; s[i].z *= al; s[i].w *= al;
    r.x += e * s[i].x; r.y += e * s[i].y; r.z += e * s[i].z; r.w += e * s[i].w;
    p.x += qc * s[i].x; p.y += qc * s[i].y; p.z += qc * s[i].z; p.w += qc * s[i].w;
  }
  *reinterpret_cast<float4*>(&s_red_r[rg][4 * j4]) = r;
  *reinterpret_cast<float4*>(&s_red_p[rg][4 * j4]) = p;
  __syncthreads();

  r = make_float4(0.f, 0.f, 0.f, 0.f);
  p = r;
  // two row groups per step: unrolled fully, the compiler holds every partial at
  // once beside the state rows (64 more VGPRs, one workgroup fewer per CU)
#pragma unroll 2
  for (int g = 0; g < RG; ++g) {
    const float4 x = *reinterpret_cast<const float4*>(&s_red_r[g][4 * j4]);
    const float4 y = *reinterpret_cast<const float4*>(&s_red_p[g][4 * j4]);
    r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
    p.x += y.x; p.y += y.y; p.z += y.z; p.w += y.w;
  }
  float kqs = 0.f;
#pragma unroll
  for (int wv = 0; wv < NWAVES; ++wv) kqs += s_wsum[wv];

  if (a.raw_gates) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wg[e] = sigmoid_f(wg[e]);
  }
  const float4 u = make_float4(wg[0] * vv[0] - r.x, wg[1] * vv[1] - r.y, wg[2] * vv[2] - r.z, wg[3] * vv[3] - r.w);
  if (rg == 0) {
    *reinterpret_cast<float4*>(a.o + vec_v + 4 * j4) =
        make_float4(p.x + kqs * u.x, p.y + kqs * u.y, p.z + kqs * u.z, p.w + kqs * u.w);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * row_of(i);
    const float kc = s_k[c];
    const float4 n = make_float4(s[i].x + kc * u.x, s[i].y + kc * u.y, s[i].z + kc * u.z, s[i].w + kc * u.w);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, n), Sr, voff, row_of(i) * kRowStep, 0);
  }
}

template <int DK, int DV, bool F32IN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  using Sh = DecodeShape<DK, DV>;
  hipLaunchKernelGGL((gdn2_decode_kernel<DK, DV, F32IN>), dim3(a.B * a.H), dim3(Sh::kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DK, bool F32IN>
static hipError_t launch_decode_dv(const DecodeArgs& a, hipStream_t s) {
  switch (a.Dv) {
    case 16: return launch_decode_t<DK, 16, F32IN>(a, s);
    case 32: return launch_decode_t<DK, 32, F32IN>(a, s);
    case 64: return launch_decode_t<DK, 64, F32IN>(a, s);
    case 128: return launch_decode_t<DK, 128, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_decode_dk(const DecodeArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_decode_dv<16, F32IN>(a, s);
    case 32: return launch_decode_dv<32, F32IN>(a, s);
    case 64: return launch_decode_dv<64, F32IN>(a, s);
    case 128: return launch_decode_dv<128, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.f32_inputs ? launch_decode_dk<true>(a, stream) : launch_decode_dk<false>(a, stream);
}

}  // namespace gdn2
