// gdn2_prep.hip -- chunk-parallel half of the two-stage chunkwise forward:
// everything of a chunk that does not depend on the state entering it.
//
// For a chunk of C tokens (local index r, in-chunk cumulative log-decay
// g_r = sum_{i<=r} log_alpha_i, g_C its value at the last token) the chunkwise
// WY form of the Gated Delta Rule-2 recurrence (arXiv 2605.22791 abstract:
// asymmetric key-/value-selective erase and write with channel-wise decay;
// research-wiki summary, "Key findings") needs
//   Kh = exp(g) * b * k,  Kt = k * exp(-g),
//   A  = strict_lower(Kh Kt^T),  T = (I + A)^-1,
//   W  = T Kh,  Ut = T (w * v),  P = lower_incl((q exp(g)) Kt^T),
//   Qs = q exp(g),  Kb = k exp(g_C - g),  gamma = exp(g_C),
// after which the chain only has U = Ut - W S, O = Qs S + P U and
// S <- Diag(gamma) S + Kb^T U left (the state-dependent part). One workgroup
// computes one (batch, head, chunk): all B*H*ceil(T/C) chunks run in parallel.
//
// Outputs (workspace): the record of units -W, Qs, Kb^T, P, gamma (see
// gdn2_frag.h) and Ut as fp32 accumulator tiles: tile (R, jb) of 16 x 16 at
// float offset 256 * (R * Dv/16 + jb), lane l's 4 values (rows 4(l/16)+i,
// column l%16) contiguous, so the chain reads each tile with one 16-byte load
// per lane.
//
// Precision as in the single-pass forward: A and P from a two-term bf16 split
// of their decay-scaled factors (referenced to the chunk middle so that the
// exp(+-g) factors stay in range), all other operands fp16 for bf16 inputs;
// fp32 matrix cores for fp32 inputs.

#include "gdn2_chunk.h"
#include "gdn2_frag.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <int DK, int C, bool F32IN>
struct PrepCfg {
  static constexpr int kThreads = 512;
  using KS = KSide<DK, C, F32IN, kThreads>;
  using OpT = typename KS::OpT;
  using Rec = Record<DK, C, F32IN, 0>;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int NB = KS::NB;
  static constexpr int LDC = KS::LDC, LDK = KS::LDK, LDCF = KS::LDCF;
  static constexpr int OPB = sizeof(OpT);
  static constexpr int DVM = 128;                                  // largest value width
  // persistent region
  static constexpr int oKhT = 0;                                   // OpT [DK][LDC]  (b k exp(g))^T
  static constexpr int oQs = oKhT + DK * LDC * OPB;                // OpT [C][LDK]   q exp(g)
  static constexpr int oKbT = oQs + C * LDK * OPB;                 // OpT [DK][LDC]  (k exp(g_C - g))^T
  static constexpr int oCH = oKbT + DK * LDC * OPB;                // float [4][DK]
  static constexpr int oTOT = oCH + KS::kChanBytes;
  static constexpr int oX = oTOT + KS::kTotBytes;
  // phase F
  static constexpr int oG = oX;
  static constexpr int oSL = oG + KS::kGBytes;
  static constexpr int endF = oSL + KS::kSlicesBytes;
  // phase W
  static constexpr int oAf = oX;                                   // float [C][LDCF]  A, then T
  static constexpr int oPm = oAf + KS::kAfBytes;                   // OpT [C][LDC]     P
  static constexpr int oWVT = oPm + C * LDC * OPB;                 // OpT [DVM][LDC]   (w v)^T
  static constexpr int oXs = oWVT + DVM * LDC * OPB;
  static constexpr int endW = oXs + KS::kXsBytes;
  static constexpr int kLdsBytes = endF > endW ? endF : endW;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;
  // v, w: 8 consecutive value columns of one row, up to DVM columns
  static constexpr int VW_PT = (C * DVM / 8 + kThreads - 1) / kThreads;
};

template <int DK, int C, bool F32IN>
__global__ __launch_bounds__(512) void gdn2_prep_fwd_kernel(FwdArgs a, char* rec_base, float* ut_base) {
  using Cfg = PrepCfg<DK, C, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  using Rec = typename Cfg::Rec;
  using F = Frag<F32IN>;
  constexpr int NW = Cfg::kWaves, NB = Cfg::NB, NT = Cfg::kThreads;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDCF = Cfg::LDCF;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  OpT* sKhT = reinterpret_cast<OpT*>(smem + Cfg::oKhT);
  OpT* sQs = reinterpret_cast<OpT*>(smem + Cfg::oQs);
  OpT* sKbT = reinterpret_cast<OpT*>(smem + Cfg::oKbT);
  float* sCh = reinterpret_cast<float*>(smem + Cfg::oCH);
  float* sTot = reinterpret_cast<float*>(smem + Cfg::oTOT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  OpT* sPm = reinterpret_cast<OpT*>(smem + Cfg::oPm);
  OpT* sWVT = reinterpret_cast<OpT*>(smem + Cfg::oWVT);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lg = l >> 4;

  const int Dv = a.Dv, T = a.T, H = a.H;
  const int NC = (T + C - 1) / C;
  // block -> (batch*head, chunk), chunk fastest
  const int bh = blockIdx.x / NC, n = blockIdx.x - bh * NC;
  const int bi = bh / H, h = bh - bi * H;
  const int t0 = n * C, Lr = min(C, T - t0);
  const int64_t rowK = (int64_t)H * DK, rowV = (int64_t)H * Dv;
  const int64_t baseK = ((int64_t)bi * T * H + h) * DK;
  const int64_t baseV = ((int64_t)bi * T * H + h) * Dv;
  char* rec = rec_base + ((int64_t)bh * NC + n) * Rec::kBytes;
  float* ut = ut_base + ((int64_t)bh * NC + n) * C * Dv;

  KS ks;
  ks.init(tid);
  ks.load(a.q, a.k, a.b, a.log_alpha, baseK, rowK, t0, Lr);
  const int vpr = Dv / 8;  // threads per row of v, w
  Raw8<F32IN> rv[Cfg::VW_PT], rw[Cfg::VW_PT];
#pragma unroll
  for (int i = 0; i < Cfg::VW_PT; ++i) {
    const int e = tid + NT * i, r = e / vpr, j8 = e - r * vpr;
    if (r < Lr) {
      const int64_t idx = baseV + (int64_t)(t0 + r) * rowV + 8 * j8;
      ld_raw(rv[i], a.v, idx);
      ld_raw(rw[i], a.w, idx);
    } else {
      zero_raw(rv[i]);
      zero_raw(rw[i]);
    }
  }

  // ---- gates, factors, Gram products ----
  ks.gates(sTot, sG, sCh);
  f32x4 accG[KS::GPW];
  ks.factors_gram(sG, sCh, sSL, accG,
                  [&](int r, int c0, const float (&qv)[4], const float (&kv)[4], const float (&bv)[4],
                      const float (&e1)[4], const float (&eg)[4], const float (&ec)[4]) {
                    (void)e1;
                    st4(sQs + r * LDK + c0, qv[0] * eg[0], qv[1] * eg[1], qv[2] * eg[2], qv[3] * eg[3]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                      sKhT[(c0 + i) * LDC + r] = static_cast<OpT>(bv[i] * kv[i] * eg[i]);
                      sKbT[(c0 + i) * LDC + r] = static_cast<OpT>(kv[i] * ec[i]);
                    }
                  });
  ks.template gram_store<false>(accG, sAf, sPm);
  // (w v)^T: the Gram slices are dead now
#pragma unroll
  for (int i = 0; i < Cfg::VW_PT; ++i) {
    const int e = tid + NT * i, r = e / vpr, j8 = e - r * vpr;
    if (r < C) {
      float vv[8], ww[8];
      cvt(rv[i], vv);
      cvt(rw[i], ww);
#pragma unroll
      for (int q = 0; q < 8; ++q) sWVT[(8 * j8 + q) * LDC + r] = static_cast<OpT>(ww[q] * vv[q]);
    }
  }
  ks.invert(sAf, sXs);  // begins and ends with a barrier

  // ---- record: -W (from W^T tiles), Qs, Kb^T, P, gamma ----
  {
    // unit (R, u) of -W pairs the W^T tiles of channel blocks 2u, 2u+1 (16-bit)
    // or is the tile of channel block u (fp32)
    constexpr int CPU = F32IN ? 1 : 2;  // channel tiles per unit
    constexpr int NWU = (C / 16) * Rec::UK;
    for (int t = wid; t < NWU; t += NW) {
      const int R = t / Rec::UK, u = t - R * Rec::UK;
      f32x4 w2[CPU];
#pragma unroll
      for (int p = 0; p < CPU; ++p) {
        w2[p] = zero4();
        const int cb = CPU * u + p;
        if (cb < DK / 16) mma_nt_yf32<OpT>(w2[p], sKhT + 16 * cb * LDC, LDC, sAf + 16 * R * LDCF, LDCF, 16 * (R + 1));
      }
      uint4 out;
      if constexpr (F32IN) {
        out = make_uint4(__float_as_uint(-w2[0][0]), __float_as_uint(-w2[0][1]), __float_as_uint(-w2[0][2]),
                         __float_as_uint(-w2[0][3]));
      } else {
        f16x8 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[i] = static_cast<_Float16>(-w2[0][i]);
          hv[4 + i] = static_cast<_Float16>(-w2[CPU - 1][i]);
        }
        out = __builtin_bit_cast(uint4, hv);
      }
      *reinterpret_cast<uint4*>(rec + (int64_t)(Rec::u0 + t) * F::kUnitBytes + 16 * l) = out;
    }
    write_units<F32IN>(sQs, LDK, C, DK, rec + Rec::u1 * F::kUnitBytes, wid, NW);
    write_units<F32IN>(sKbT, LDC, DK, C, rec + Rec::u2 * F::kUnitBytes, wid, NW);
    write_units<F32IN>(sPm, LDC, C, C, rec + Rec::u3 * F::kUnitBytes, wid, NW);
    float* gam = reinterpret_cast<float*>(rec + Rec::uG * F::kUnitBytes);
    for (int c = tid; c < DK; c += NT) gam[c] = __expf(sCh[DK + c]);
  }

  // ---- Ut = T (w v): accumulator tiles straight to the workspace ----
  {
    const int nvt = Dv / 16, ntile = (C / 16) * nvt;
    for (int t = wid; t < ntile; t += NW) {
      const int R = t / nvt, jb = t - R * nvt;
      f32x4 acc = zero4();
      mma_nt_xf32<OpT>(acc, sAf + 16 * R * LDCF, LDCF, sWVT + 16 * jb * LDC, LDC, 16 * (R + 1));
      *reinterpret_cast<float4*>(ut + (int64_t)t * 256 + 4 * l) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
  (void)lg;
}

template <int DK, int C, bool F32IN>
static hipError_t launch_prep_fwd_t(const FwdArgs& a, char* rec, float* ut, hipStream_t s) {
  if constexpr (!PrepCfg<DK, C, F32IN>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int NC = (a.T + C - 1) / C;
    const int64_t grid = (int64_t)a.B * a.H * NC;
    hipLaunchKernelGGL((gdn2_prep_fwd_kernel<DK, C, F32IN>), dim3((unsigned)grid), dim3(512), 0, s, a, rec, ut);
    return hipGetLastError();
  }
}

template <int DK, bool F32IN>
static hipError_t launch_prep_fwd_c(const FwdArgs& a, char* rec, float* ut, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_prep_fwd_t<DK, 16, F32IN>(a, rec, ut, s);
    case 32: return launch_prep_fwd_t<DK, 32, F32IN>(a, rec, ut, s);
    case 64: return launch_prep_fwd_t<DK, 64, F32IN>(a, rec, ut, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_prep_fwd_f(const FwdArgs& a, char* rec, float* ut, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_prep_fwd_c<16, F32IN>(a, rec, ut, s);
    case 32: return launch_prep_fwd_c<32, F32IN>(a, rec, ut, s);
    case 64: return launch_prep_fwd_c<64, F32IN>(a, rec, ut, s);
    case 128: return launch_prep_fwd_c<128, F32IN>(a, rec, ut, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prep_fwd(const FwdArgs& a, char* rec, float* ut, hipStream_t s) {
  return a.f32_inputs ? launch_prep_fwd_f<true>(a, rec, ut, s) : launch_prep_fwd_f<false>(a, rec, ut, s);
}

template <int DK, bool F32IN>
static bool prep_fits_c(int chunk) {
  switch (chunk) {
    case 16: return PrepCfg<DK, 16, F32IN>::kFits;
    case 32: return PrepCfg<DK, 32, F32IN>::kFits;
    case 64: return PrepCfg<DK, 64, F32IN>::kFits;
  }
  return false;
}

bool prep_fwd_supported(int Dk, int chunk, bool f32) {
  switch (Dk) {
    case 16: return f32 ? prep_fits_c<16, true>(chunk) : prep_fits_c<16, false>(chunk);
    case 32: return f32 ? prep_fits_c<32, true>(chunk) : prep_fits_c<32, false>(chunk);
    case 64: return f32 ? prep_fits_c<64, true>(chunk) : prep_fits_c<64, false>(chunk);
    case 128: return f32 ? prep_fits_c<128, true>(chunk) : prep_fits_c<128, false>(chunk);
  }
  return false;
}

size_t fwd_record_bytes(int Dk, int chunk, bool f32) {
#define GDN2_REC(DK, CC)                                                              \
  if (Dk == DK && chunk == CC)                                                        \
    return f32 ? (size_t)Record<DK, CC, true, 0>::kBytes : (size_t)Record<DK, CC, false, 0>::kBytes;
  GDN2_REC(16, 16) GDN2_REC(16, 32) GDN2_REC(16, 64)
  GDN2_REC(32, 16) GDN2_REC(32, 32) GDN2_REC(32, 64)
  GDN2_REC(64, 16) GDN2_REC(64, 32) GDN2_REC(64, 64)
  GDN2_REC(128, 16) GDN2_REC(128, 32) GDN2_REC(128, 64)
#undef GDN2_REC
  return 0;
}

}  // namespace gdn2
