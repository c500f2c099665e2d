// gdn2_bwd.hip -- gate-aware chunkwise backward of the Gated Delta Rule-2 operator.
//
// Gradients of L = <dO, o> + <dS_final, S_T> with respect to q, k, v, log_alpha,
// b, w and S0 (the gate-aware backward of arXiv 2605.22791 abstract and the
// aiexpert.news method paragraph). Per chunk (notation of gdn2_fwd.hip; S0 is
// the chunk's entry state, dS the gradient of its exit state):
//
//   U      = T (w*v - Kh S0)
//   dU     = P^T dO + Kb dS
//   dS0    = Qs^T dO + Diag(exp(g_C)) dS - Kh^T T^T dU           (carried to the previous chunk)
//   dP     = lower_incl(dO U^T)          dQs = dO S0^T            dKb = U dS^T
//   dW     = -dU S0^T                    dT  = dW Kh^T + dU (w*v)^T
//   d(w*v) = T^T dU                      dA  = strict_lower(-T^T dT T^T)
//   dKh    = T^T dW      dKh' = dA Kt'   dQh' = dP Kt'            dKt' = dA^T Kh' + dP^T Qh'
//
// with Kh, Qs, Kb referenced to the chunk start and Kh', Qh', Kt' to the chunk
// middle (the Gram factors). Chain rule through the elementwise factors:
//   dq = dQs exp(g) + dQh' exp(g - g_m)
//   db = k (dKh exp(g) + dKh' exp(g - g_m))
//   dk = b (dKh exp(g) + dKh' exp(g - g_m)) + dKt' exp(g_m - g) + dKb exp(g_C - g)
//   dw = d(w*v) v,  dv = d(w*v) w.
// The decay gradient needs no differentiation through the exp factors: the
// operator is invariant under q/l, l k, b/l^2, S l on the key axis, which gives
//   dlog_alpha_t = sum_{s >= t in chunk} (q dq + 2 b db - k dk)_s + rowsum(S_exit * dS)
//   rowsum(S_exit * dS) = exp(g_C) rowsum(S0 * dS) + colsum_r(Kb * dKb).
//
// Two kernels:
//   * gdn2_bwd_dstate_kernel: one workgroup per (batch, head, value tile), chunks
//     in reverse; carries dS (value columns are independent) and stores the exit
//     gradient of every chunk; its final carry is dS0.
//   * gdn2_bwd_grad_kernel: one workgroup per (batch, head, chunk), fully
//     parallel; loops over value tiles accumulating the key-side partial
//     products in registers, then forms every gradient of the chunk.
// Precision as in the forward: fp16 operands with fp32 accumulation, and a
// two-term bf16 split for the products with the wide-range factors Kh', Qh', Kt'.

#include "gdn2_chunk.h"
#include "gdn2_frag.h"
#include "gdn2_internal.h"

namespace gdn2 {

// =============================================================================
// reverse state-gradient chain
// =============================================================================
// Reverse chain: 8 waves per workgroup, as in the forward.
constexpr int kDstThreads = 512;

template <int DK, int C, int BV, bool F32IN>
struct DstCfg {
  static constexpr int kThreads = kDstThreads;
  using KS = KSide<DK, C, F32IN, kThreads>;
  using OpT = typename KS::OpT;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int NB = KS::NB;
  static constexpr int LDC = KS::LDC, LDK = KS::LDK, LDCF = KS::LDCF;
  static constexpr int OPB = sizeof(OpT);
  static constexpr int oKhT = 0;                                   // OpT [DK][LDC]  (b k exp(g))^T
  static constexpr int oQhT = oKhT + DK * LDC * OPB;               // OpT [DK][LDC]  (q exp(g))^T
  static constexpr int oKb = oQhT + DK * LDC * OPB;                // OpT [C][LDK]   k exp(g_C - g)
  static constexpr int oDOT = oKb + C * LDK * OPB;                 // OpT [BV][LDC]  dO^T
  static constexpr int oDST = oDOT + BV * LDC * OPB;               // OpT [BV][LDK]  dS^T
  static constexpr int oCH = oDST + BV * LDK * OPB;
  static constexpr int oTOT = oCH + KS::kChanBytes;
  static constexpr int oX = oTOT + KS::kTotBytes;
  static constexpr int oG = oX;
  static constexpr int oSL = oG + KS::kGBytes;
  static constexpr int endF = oSL + KS::kSlicesBytes;
  static constexpr int oAf = oX;                                   // float [C][LDCF] T
  static constexpr int oPT = oAf + KS::kAfBytes;                   // OpT [C][LDC]   P^T
  static constexpr int oTT = oPT + C * LDC * OPB;                  // OpT [C][LDC]   T^T
  static constexpr int oDUT = oTT + C * LDC * OPB;                 // OpT [BV][LDC]  dU^T
  static constexpr int oZT = oDUT + BV * LDC * OPB;                // OpT [BV][LDC]  -(T^T dU)^T
  static constexpr int oXs = oZT + BV * LDC * OPB;
  static constexpr int endW = oXs + KS::kXsBytes;
  static constexpr int kLdsBytes = endF > endW ? endF : endW;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;
  static constexpr int NUT = NB * (BV / 16);
  static constexpr int UPW = (NUT + kWaves - 1) / kWaves;
  static constexpr int NST = (DK / 16) * (BV / 16);
  static constexpr int SPW = (NST + kWaves - 1) / kWaves;
  static constexpr int VW_RPP = kThreads / (BV / 8);
  static constexpr int VW_RPT = (C + VW_RPP - 1) / VW_RPP;
};

template <int DK, int C, int BV, bool F32IN>
__global__ __launch_bounds__(kDstThreads) void gdn2_bwd_dstate_kernel(BwdArgs a) {
  using Cfg = DstCfg<DK, C, BV, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  constexpr int NW = Cfg::kWaves, NB = Cfg::NB, NT = Cfg::kThreads;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDCF = Cfg::LDCF;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  OpT* sKhT = reinterpret_cast<OpT*>(smem + Cfg::oKhT);
  OpT* sQhT = reinterpret_cast<OpT*>(smem + Cfg::oQhT);
  OpT* sKb = reinterpret_cast<OpT*>(smem + Cfg::oKb);
  OpT* sDOT = reinterpret_cast<OpT*>(smem + Cfg::oDOT);
  OpT* sDST = reinterpret_cast<OpT*>(smem + Cfg::oDST);
  float* sCh = reinterpret_cast<float*>(smem + Cfg::oCH);
  float* sTot = reinterpret_cast<float*>(smem + Cfg::oTOT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  OpT* sPT = reinterpret_cast<OpT*>(smem + Cfg::oPT);
  OpT* sTT = reinterpret_cast<OpT*>(smem + Cfg::oTT);
  OpT* sDUT = reinterpret_cast<OpT*>(smem + Cfg::oDUT);
  OpT* sZT = reinterpret_cast<OpT*>(smem + Cfg::oZT);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int nv = a.Dv / BV;
  const int nbh = a.B * a.H;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int bh = (slot / nv) * 8 + xcd, vt = slot % nv;
  if (bh >= nbh) return;
  const int bi = bh / a.H, h = bh - bi * a.H;
  const int j0 = vt * BV;
  const int Dv = a.Dv, T = a.T, H = a.H;
  const int NC = (T + C - 1) / C;
  const int64_t rowK = (int64_t)H * DK, rowV = (int64_t)H * Dv;
  const int64_t baseK = ((int64_t)bi * T * H + h) * DK;
  const int64_t baseV = ((int64_t)bi * T * H + h) * Dv + j0;
  const int64_t stBase = (int64_t)bh * DK * Dv + j0;

  KS ks;
  ks.init(tid);
  constexpr int VW_RPP = Cfg::VW_RPP, VW_RPT = Cfg::VW_RPT;
  const int vw_r = tid / (BV / 8), vw_j8 = tid % (BV / 8);
  Raw8<F32IN> rdo[VW_RPT];
  auto load_chunk = [&](int nn) {
    const int tn = nn * C, Ln = min(C, T - tn);
    ks.load(a.q, a.k, a.b, a.log_alpha, baseK, rowK, tn, Ln);
#pragma unroll
    for (int i = 0; i < VW_RPT; ++i) {
      const int r = vw_r + i * VW_RPP;
      if (r < Ln) ld_raw(rdo[i], a.dO, baseV + (int64_t)(tn + r) * rowV + 8 * vw_j8);
      else zero_raw(rdo[i]);
    }
  };

  // dS starts as dS_final (or zero)
  f32x4 accD[Cfg::SPW];
#pragma unroll
  for (int i = 0; i < Cfg::SPW; ++i) {
    const int t = wid + NW * i;
    accD[i] = zero4();
    if (t < Cfg::NST) {
      const int cb = t / (BV / 16), jb = t % (BV / 16);
      if (a.dS_final) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accD[i][e] = a.dS_final[stBase + (int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr];
      }
      store_tile_t(sDST + 16 * jb * LDK + 16 * cb, LDK, accD[i]);
    }
  }
  load_chunk(NC - 1);

  for (int n = NC - 1; n >= 0; --n) {
    // the carried gradient is that of chunk n's exit state
    {
      float* ws = a.dS_chunks + ((int64_t)bh * NC + n) * DK * Dv + j0;
#pragma unroll
      for (int i = 0; i < Cfg::SPW; ++i) {
        const int t = wid + NW * i;
        if (t < Cfg::NST) {
          const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) ws[(int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr] = accD[i][e];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < VW_RPT; ++i) {
      const int r = vw_r + i * VW_RPP;
      if (r < C) {
        float d8[8];
        cvt(rdo[i], d8);
#pragma unroll
        for (int e = 0; e < 8; ++e) sDOT[(8 * vw_j8 + e) * LDC + r] = static_cast<OpT>(d8[e]);
      }
    }
    ks.gates(sTot, sG, sCh);
    f32x4 accG[KS::GPW];
    ks.factors_gram(sG, sCh, sSL, accG,
                    [&](int r, int c0, const float (&qv)[4], const float (&kv)[4], const float (&bv)[4],
                        const float (&e1)[4], const float (&eg)[4], const float (&ec)[4]) {
                      (void)e1;
                      st4(sKb + r * LDK + c0, kv[0] * ec[0], kv[1] * ec[1], kv[2] * ec[2], kv[3] * ec[3]);
#pragma unroll
                      for (int i = 0; i < 4; ++i) {
                        sKhT[(c0 + i) * LDC + r] = static_cast<OpT>(bv[i] * kv[i] * eg[i]);
                        sQhT[(c0 + i) * LDC + r] = static_cast<OpT>(qv[i] * eg[i]);
                      }
                    });
    ks.template gram_store<true>(accG, sAf, sPT);
    ks.invert(sAf, sXs);
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      sTT[i * LDC + r] = static_cast<OpT>(sAf[r * LDCF + i]);
    }
    if (n > 0) load_chunk(n - 1);
    __syncthreads();

    // dU = P^T dO + Kb dS
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NUT) {
        const int R = t / (BV / 16), jb = t % (BV / 16);
        f32x4 acc = zero4();
        mma_nt<OpT>(acc, sPT + 16 * R * LDC + 16 * R, LDC, sDOT + 16 * jb * LDC + 16 * R, LDC, C - 16 * R);
        mma_nt_k<DK>(acc, sKb + 16 * R * LDK, LDK, sDST + 16 * jb * LDK, LDK);
        store_tile_t(sDUT + 16 * jb * LDC + 16 * R, LDC, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // Z = T^T dU, stored negated
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NUT) {
        const int I = t / (BV / 16), jb = t % (BV / 16);
        f32x4 acc = zero4();
        mma_nt<OpT>(acc, sTT + 16 * I * LDC + 16 * I, LDC, sDUT + 16 * jb * LDC + 16 * I, LDC, C - 16 * I);
        store_tile_t(sZT + 16 * jb * LDC + 16 * I, LDC, acc, -1.f);
      }
    }
    __syncthreads();
    // dS <- Diag(exp(g_C)) dS + Qs^T dO - Kh^T Z
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NST) {
        const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) accD[i][e] *= __expf(sCh[DK + 16 * cb + 4 * lg + e]);
        mma_nt_k<C>(accD[i], sQhT + 16 * cb * LDC, LDC, sDOT + 16 * jb * LDC, LDC);
        mma_nt_k<C>(accD[i], sKhT + 16 * cb * LDC, LDC, sZT + 16 * jb * LDC, LDC);
        store_tile_t(sDST + 16 * jb * LDK + 16 * cb, LDK, accD[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (a.dS0) {
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NST) {
        const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) a.dS0[stBase + (int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr] = accD[i][e];
      }
    }
  }
}

// =============================================================================
// chunk-parallel gradients
// =============================================================================

// Four input values kept in registers: fp32 as is, bf16 as two packed pairs
// (exact: the inputs are bf16 numbers).
template <bool F32IN>
struct Vals4 {
  float v[4];
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
  __device__ __forceinline__ void set(int e, const void* base, int64_t idx) {
    v[e] = static_cast<const float*>(base)[idx];
  }
  __device__ __forceinline__ float operator[](int e) const { return v[e]; }
};
template <>
struct Vals4<false> {
  uint32_t p[2];
  __device__ __forceinline__ void zero() { p[0] = p[1] = 0u; }
  __device__ __forceinline__ void set(int e, const void* base, int64_t idx) {
    const uint32_t x = static_cast<const uint16_t*>(base)[idx];
    p[e >> 1] = (e & 1) ? ((p[e >> 1] & 0x0000ffffu) | (x << 16)) : ((p[e >> 1] & 0xffff0000u) | x);
  }
  __device__ __forceinline__ float operator[](int e) const {
    return __uint_as_float((e & 1) ? (p[e >> 1] & 0xffff0000u) : (p[e >> 1] << 16));
  }
};
template <int DK, int C, int BVB_, bool F32IN>
struct GradCfg {
  using KS = KSide<DK, C, F32IN, 512, 4>;  // float4 log_alpha rows: the decay-gradient scan reuses them
  using OpT = typename KS::OpT;
  // operand type of the products with the wide-range Gram factors: a bf16 hi/lo
  // pair for bf16 inputs, fp32 for fp32 inputs
  using WideT = typename std::conditional<F32IN, float, __bf16>::type;
  static constexpr int WPARTS = F32IN ? 1 : 2;
  static constexpr int kThreads = 512;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int NB = KS::NB;
  static constexpr int BVB = BVB_;                                 // value tile of the inner loop
  static constexpr int LDC = KS::LDC, LDK = KS::LDK, LDCF = KS::LDCF;
  static constexpr int LDB = BVB + KS::PADOP;                      // rows of BVB values
  static constexpr int OPB = sizeof(OpT);
  static constexpr int WB = sizeof(WideT);
  // persistent (until the post-processing)
  static constexpr int oKh = 0;                                    // OpT [C][LDK]  b k exp(g)
  static constexpr int oKb = oKh + C * LDK * OPB;                  // OpT [C][LDK]  k exp(g_C - g)
  static constexpr int oTm = oKb + C * LDK * OPB;                  // OpT [C][LDC]  T
  static constexpr int oTT = oTm + C * LDC * OPB;                  // OpT [C][LDC]  T^T
  static constexpr int oPT = oTT + C * LDC * OPB;                  // OpT [C][LDC]  P^T
  static constexpr int oR = oPT + C * LDC * OPB;                   // phase region
  // phase F / T (prep)
  static constexpr int oG = oR;
  static constexpr int oSL = oG + KS::kGBytes;
  static constexpr int endPF = oSL + KS::kSlicesBytes;
  static constexpr int oAf = oR;
  static constexpr int oXs = oAf + KS::kAfBytes;
  static constexpr int endPT = oXs + KS::kXsBytes;
  // phase V (value-tile loop)
  static constexpr int oS0T = oR;                                  // OpT [BVB][LDK]
  static constexpr int oS0 = oS0T + BVB * LDK * OPB;               // OpT [DK][LDB]
  static constexpr int oDST = oS0 + DK * LDB * OPB;                // OpT [BVB][LDK]
  static constexpr int oDS = oDST + BVB * LDK * OPB;               // OpT [DK][LDB]
  static constexpr int oDO = oDS + DK * LDB * OPB;                 // OpT [C][LDB]
  static constexpr int oDOT = oDO + C * LDB * OPB;                 // OpT [BVB][LDC]
  static constexpr int oWV = oDOT + BVB * LDC * OPB;               // OpT [C][LDB]
  static constexpr int oXT = oWV + C * LDB * OPB;                  // OpT [BVB][LDC]
  static constexpr int oU = oXT + BVB * LDC * OPB;                 // OpT [C][LDB]
  static constexpr int oDU = oU + C * LDB * OPB;                   // OpT [C][LDB]
  static constexpr int oDUT = oDU + C * LDB * OPB;                 // OpT [BVB][LDC]
  static constexpr int endV = oDUT + BVB * LDC * OPB;
  // phase A (dT, dK, dA)
  static constexpr int oDW = oR;                                   // OpT [C][LDK]
  static constexpr int oDWT = oDW + C * LDK * OPB;                 // OpT [DK][LDC]
  static constexpr int oDTm = oDWT + DK * LDC * OPB;               // OpT [C][LDC]
  static constexpr int oMT = oDTm + C * LDC * OPB;                 // OpT [C][LDC]
  static constexpr int endA = oMT + C * LDC * OPB;
  // phase B (wide-range products) starts at 0: every earlier buffer is dead
  static constexpr int kWM = C * LDC * WB;                         // one part of a [C][LDC] wide matrix
  static constexpr int oWdA = 0;                                   // dA, dA^T, dP, dP^T (hi/lo or fp32)
  static constexpr int oWF = oWdA + 4 * WPARTS * kWM;              // factor^T [DK][LDC] (hi/lo or fp32)
  static constexpr int endB = oWF + WPARTS * DK * LDC * WB;
  // phase D (output staging and the decay-gradient scan) starts at 0 as well:
  // x, and where they fit, dq, dk, db as fp32 [C][DK] (staged for full-row stores)
  static constexpr int endBase = [] {
    int m = endPF;
    if (endPT > m) m = endPT;
    if (endV > m) m = endV;
    if (endA > m) m = endA;
    if (endB > m) m = endB;
    return m;
  }();
  // cumsum segment totals: scratch of the gate prep and of the final scan only,
  // so they sit past the prep buffers and the output staging
  static constexpr int tot_at(int endD_) { return ((endPF > endD_ ? endPF : endD_) + 15) & ~15; }
  static constexpr int main_end(int endD_) {
    return endBase > tot_at(endD_) + KS::kTotBytes ? endBase : tot_at(endD_) + KS::kTotBytes;
  }
  static constexpr int kTail = KS::kChanBytes + 2 * DK * 4 + kWaves * DK * 4;
  static constexpr bool kStage = ((main_end(4 * C * DK * 4) + 15) & ~15) + kTail <= 160 * 1024;
  static constexpr int endD = (kStage ? 4 : 1) * C * DK * 4;
  static constexpr int oTOT = tot_at(endD);
  static constexpr int endMain = main_end(endD);
  // tail (always live)
  static constexpr int oCH = (endMain + 15) & ~15;
  static constexpr int oEX = oCH + KS::kChanBytes;                 // float [2][DK] exit-term pieces
  static constexpr int oEXW = oEX + 2 * DK * 4;                    // float [kWaves][DK] per-wave partials
  static constexpr int kLdsBytes = oEXW + kWaves * DK * 4;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;

  static constexpr int NKT = NB * (DK / 16);                       // C x DK tiles
  static constexpr int KPW = (NKT + kWaves - 1) / kWaves;
  static constexpr int NCT = NB * NB;                              // C x C tiles
  static constexpr int CPW = (NCT + kWaves - 1) / kWaves;
  static constexpr int NVT = NB * (BVB / 16);                      // C x BVB tiles
  static constexpr int VPW = (NVT + kWaves - 1) / kWaves;
};

// REC: T and P^T come from the backward records (a.records) and the chunk's
// Gram products and inversion are skipped; otherwise they are recomputed here.
template <int DK, int C, int BVB_, bool F32IN, bool REC>
__global__ __launch_bounds__(512) void gdn2_bwd_grad_kernel(BwdArgs a) {
  using Cfg = GradCfg<DK, C, BVB_, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  using WideT = typename Cfg::WideT;
  constexpr int NW = Cfg::kWaves, NB = Cfg::NB, NT = Cfg::kThreads, BVB = Cfg::BVB;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDCF = Cfg::LDCF, LDB = Cfg::LDB;
  constexpr int KPW = Cfg::KPW, CPW = Cfg::CPW, VPW = Cfg::VPW;
  constexpr int KB16 = DK / 16, VB16 = BVB / 16;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  OpT* sKh = reinterpret_cast<OpT*>(smem + Cfg::oKh);
  OpT* sKb = reinterpret_cast<OpT*>(smem + Cfg::oKb);
  OpT* sTm = reinterpret_cast<OpT*>(smem + Cfg::oTm);
  OpT* sTT = reinterpret_cast<OpT*>(smem + Cfg::oTT);
  OpT* sPT = reinterpret_cast<OpT*>(smem + Cfg::oPT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);
  OpT* sS0T = reinterpret_cast<OpT*>(smem + Cfg::oS0T);
  OpT* sS0 = reinterpret_cast<OpT*>(smem + Cfg::oS0);
  OpT* sDST = reinterpret_cast<OpT*>(smem + Cfg::oDST);
  OpT* sDS = reinterpret_cast<OpT*>(smem + Cfg::oDS);
  OpT* sDO = reinterpret_cast<OpT*>(smem + Cfg::oDO);
  OpT* sDOT = reinterpret_cast<OpT*>(smem + Cfg::oDOT);
  OpT* sWV = reinterpret_cast<OpT*>(smem + Cfg::oWV);
  OpT* sXT = reinterpret_cast<OpT*>(smem + Cfg::oXT);
  OpT* sU = reinterpret_cast<OpT*>(smem + Cfg::oU);
  OpT* sDU = reinterpret_cast<OpT*>(smem + Cfg::oDU);
  OpT* sDUT = reinterpret_cast<OpT*>(smem + Cfg::oDUT);
  OpT* sDW = reinterpret_cast<OpT*>(smem + Cfg::oDW);
  OpT* sDWT = reinterpret_cast<OpT*>(smem + Cfg::oDWT);
  OpT* sDTm = reinterpret_cast<OpT*>(smem + Cfg::oDTm);
  OpT* sMT = reinterpret_cast<OpT*>(smem + Cfg::oMT);
  WideT* sW = reinterpret_cast<WideT*>(smem + Cfg::oWdA);
  WideT* sWF = reinterpret_cast<WideT*>(smem + Cfg::oWF);
  float* sX = reinterpret_cast<float*>(smem);
  float* sCh = reinterpret_cast<float*>(smem + Cfg::oCH);
  float* sTot = reinterpret_cast<float*>(smem + Cfg::oTOT);
  float* sEx = reinterpret_cast<float*>(smem + Cfg::oEX);
  float* sExW = reinterpret_cast<float*>(smem + Cfg::oEXW);

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int T = a.T, H = a.H, Dv = a.Dv;
  const int NC = (T + C - 1) / C;
  const int bh = blockIdx.x / NC, n = blockIdx.x % NC;
  const int bi = bh / H, h = bh - bi * H;
  const int t0 = n * C, Lr = min(C, T - t0);
  const int64_t rowK = (int64_t)H * DK, rowV = (int64_t)H * Dv;
  const int64_t baseK = ((int64_t)bi * T * H + h) * DK;
  const int64_t baseV = ((int64_t)bi * T * H + h) * Dv;
  const int64_t stOff = ((int64_t)bh * NC + n) * DK * Dv;
  const float* S0g = a.chunk_states + stOff;
  const float* dSg = a.dS_chunks + stOff;

  // ---- key-side preparation ----
  KS ks;
  ks.init(tid);
  if constexpr (REC) ks.load_la(a.log_alpha, baseK, rowK, t0, Lr);
  else ks.load(a.q, a.k, a.b, a.log_alpha, baseK, rowK, t0, Lr);
  ks.gates(sTot, sG, sCh);

  // the C x DK tiles this lane owns: rows 16R + 4lg + e, column 16cb + lr.
  // Keep q, k, b and e1 = exp(g - g_m) there for the final chain rule.
  Vals4<F32IN> pq[KPW], pk[KPW], pb[KPW];
  float pe1[KPW][4];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    pq[i].zero();
    pk[i].zero();
    pb[i].zero();
#pragma unroll
    for (int e = 0; e < 4; ++e) pe1[i][e] = 1.f;
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        pe1[i][e] = __expf(sG[r * DK + c] - sCh[c]);
        if (r < Lr) {
          const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
          pq[i].set(e, a.q, idx);
          pk[i].set(e, a.k, idx);
          pb[i].set(e, a.b, idx);
        }
      }
    }
  }

  if constexpr (REC) {
    // Kh = b k exp(g) and Kb = k exp(g_C - g) at the lane's positions
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NKT) {
        const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          const float eg = pe1[i][e] * sCh[2 * DK + c];
          const float ec = sCh[3 * DK + c] * __builtin_amdgcn_rcpf(pe1[i][e]);
          sKh[r * LDK + c] = static_cast<OpT>(pb[i][e] * pk[i][e] * eg);
          sKb[r * LDK + c] = static_cast<OpT>(pk[i][e] * ec);
        }
      }
    }
    // T (and T^T) and P^T from the record's units; P^T units that lie wholly
    // below the diagonal are not stored (zero)
    using Rec = Record<DK, C, F32IN, 1>;
    using F = Frag<F32IN>;
    const char* rec = a.records + ((int64_t)bh * NC + n) * Rec::kBytes;
    constexpr int NU = Rec::RC * Rec::UC;
    for (int t = wid; t < 2 * NU; t += NW) {
      const bool isT = t < NU;
      const int tt = isT ? t : t - NU, R = tt / Rec::UC, u = tt - R * Rec::UC;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (isT || F::KU * u + F::KU - 1 >= 16 * R)
        v = *reinterpret_cast<const uint4*>(rec + (int64_t)((isT ? Rec::u4 : Rec::u0) + tt) * F::kUnitBytes + 16 * l);
      if (isT) unpack_unit<F32IN>(v, R, u, C, sTm, LDC, sTT, LDC);
      else unpack_unit<F32IN>(v, R, u, C, sPT, LDC, static_cast<OpT*>(nullptr), 0);
    }
  } else {
    f32x4 accG[KS::GPW];
    ks.factors_gram(sG, sCh, sSL, accG,
                    [&](int r, int c0, const float (&qv)[4], const float (&kv)[4], const float (&bv)[4],
                        const float (&e1)[4], const float (&eg)[4], const float (&ec)[4]) {
                      (void)qv;
                      (void)e1;
                      st4(sKh + r * LDK + c0, bv[0] * kv[0] * eg[0], bv[1] * kv[1] * eg[1], bv[2] * kv[2] * eg[2],
                          bv[3] * kv[3] * eg[3]);
                      st4(sKb + r * LDK + c0, kv[0] * ec[0], kv[1] * ec[1], kv[2] * ec[2], kv[3] * ec[3]);
                    });
    ks.template gram_store<true>(accG, sAf, sPT);
    ks.invert(sAf, sXs);
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      const OpT v = static_cast<OpT>(sAf[r * LDCF + i]);
      sTm[r * LDC + i] = v;
      sTT[i * LDC + r] = v;
    }
  }

  // ---- value-tile loop: U, dU, d(w*v) and the key-side partial products ----
  f32x4 aQh[KPW], aKb[KPW], aW[KPW], aP[CPW], aT[CPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) aQh[i] = aKb[i] = aW[i] = zero4();
#pragma unroll
  for (int i = 0; i < CPW; ++i) aP[i] = aT[i] = zero4();
  // state-tile thread map: channel st_c + p*SROWS, 4 columns at 4*st_j4
  constexpr int ST4 = BVB / 4;
  constexpr int SROWS = NT / ST4;                                  // channels per pass
  constexpr int SPASS = (DK + SROWS - 1) / SROWS;
  const int st_c = tid / ST4, st_j4 = tid % ST4;
  float rs[SPASS];                                                 // rowsum(S0 * dS) of those channels
#pragma unroll
  for (int p = 0; p < SPASS; ++p) rs[p] = 0.f;

  // value-tile inputs, fetched one tile ahead into registers
  constexpr int VG = C * (BVB / 4);                                // 4-value groups of dO, v, w per tile
  constexpr int VLD = (VG + NT - 1) / NT;
  float4 rS0[SPASS], rDS[SPASS];
  Raw4<F32IN> rDO[VLD], rV[VLD], rW[VLD];
  const int nvt = Dv / BVB;
  auto vload = [&](int jt) {
    const int j0 = jt * BVB;
#pragma unroll
    for (int p = 0; p < SPASS; ++p) {
      const int c = st_c + p * SROWS;
      if (c < DK) {
        rS0[p] = *reinterpret_cast<const float4*>(S0g + (int64_t)c * Dv + j0 + 4 * st_j4);
        rDS[p] = *reinterpret_cast<const float4*>(dSg + (int64_t)c * Dv + j0 + 4 * st_j4);
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int e = tid + i * NT;
      const int r = e / (BVB / 4), j4 = e % (BVB / 4);
      if (e < VG && r < Lr) {
        const int64_t idx = baseV + (int64_t)(t0 + r) * rowV + j0 + 4 * j4;
        ld_raw(rDO[i], a.dO, idx);
        ld_raw(rV[i], a.v, idx);
        ld_raw(rW[i], a.w, idx);
      } else {
        zero_raw(rDO[i]);
        zero_raw(rV[i]);
        zero_raw(rW[i]);
      }
    }
  };
  vload(0);

  for (int jt = 0; jt < nvt; ++jt) {
    const int j0 = jt * BVB;
    __syncthreads();  // previous users of the phase region are done
    // S0 and dS tiles: both layouts; rowsum(S0 * dS) partials
#pragma unroll
    for (int p = 0; p < SPASS; ++p) {
      const int c = st_c + p * SROWS;
      if (c < DK) {
        const float4 s4 = rS0[p], d4 = rDS[p];
        st4(sS0 + c * LDB + 4 * st_j4, s4.x, s4.y, s4.z, s4.w);
        st4(sDS + c * LDB + 4 * st_j4, d4.x, d4.y, d4.z, d4.w);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sS0T[(4 * st_j4 + i) * LDK + c] = static_cast<OpT>(sv[i]);
          sDST[(4 * st_j4 + i) * LDK + c] = static_cast<OpT>(dv4[i]);
        }
        rs[p] += s4.x * d4.x + s4.y * d4.y + s4.z * d4.z + s4.w * d4.w;
      }
    }
    // dO, w*v: 4 consecutive value columns of one row
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int e = tid + i * NT;
      if (e < VG) {
        const int r = e / (BVB / 4), j4 = e % (BVB / 4);
        float d4[4], v4[4], w4[4];
        cvt(rDO[i], d4);
        cvt(rV[i], v4);
        cvt(rW[i], w4);
        st4(sDO + r * LDB + 4 * j4, d4[0], d4[1], d4[2], d4[3]);
        st4(sWV + r * LDB + 4 * j4, w4[0] * v4[0], w4[1] * v4[1], w4[2] * v4[2], w4[3] * v4[3]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) sDOT[(4 * j4 + q4) * LDC + r] = static_cast<OpT>(d4[q4]);
      }
    }
    if (jt + 1 < nvt) vload(jt + 1);
    __syncthreads();
    // X = w*v - Kh S0  -> X^T
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NVT) {
        const int R = t / VB16, jb = t % VB16;
        f32x4 acc = zero4();
        mma_nt_k<DK>(acc, sKh + 16 * R * LDK, LDK, sS0T + 16 * jb * LDK, LDK);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[e] = static_cast<float>(sWV[(16 * R + 4 * lg + e) * LDB + 16 * jb + lr]) - acc[e];
        store_tile_t(sXT + 16 * jb * LDC + 16 * R, LDC, acc);
      }
    }
    __syncthreads();
    // U = T X ; dU = P^T dO + Kb dS
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NVT) {
        const int R = t / VB16, jb = t % VB16;
        f32x4 u = zero4(), du = zero4();
        mma_nt<OpT>(u, sTm + 16 * R * LDC, LDC, sXT + 16 * jb * LDC, LDC, 16 * (R + 1));
        store_tile(sU + 16 * R * LDB + 16 * jb, LDB, u);
        mma_nt<OpT>(du, sPT + 16 * R * LDC + 16 * R, LDC, sDOT + 16 * jb * LDC + 16 * R, LDC, C - 16 * R);
        mma_nt_k<DK>(du, sKb + 16 * R * LDK, LDK, sDST + 16 * jb * LDK, LDK);
        store_tile(sDU + 16 * R * LDB + 16 * jb, LDB, du);
        store_tile_t(sDUT + 16 * jb * LDC + 16 * R, LDC, du);
      }
    }
    __syncthreads();
    // d(w*v) = T^T dU  -> dw, dv
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NVT) {
        const int R = t / VB16, jb = t % VB16;
        f32x4 acc = zero4();
        mma_nt<OpT>(acc, sTT + 16 * R * LDC + 16 * R, LDC, sDUT + 16 * jb * LDC + 16 * R, LDC, C - 16 * R);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          if (r < Lr) {
            const int64_t idx = baseV + (int64_t)(t0 + r) * rowV + j0 + 16 * jb + lr;
            const float vv = load1<F32IN>(a.v, idx), wv = load1<F32IN>(a.w, idx);
            a.dw[idx] = acc[e] * vv;
            a.dv[idx] = acc[e] * wv;
          }
        }
      }
    }
    // key-side partials: dO S0^T, U dS^T, dU S0^T (C x DK);  dO U^T, dU (w*v)^T (C x C)
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NKT) {
        const int R = t / KB16, cb = t % KB16;
        mma_nt_k<BVB>(aQh[i], sDO + 16 * R * LDB, LDB, sS0 + 16 * cb * LDB, LDB);
        mma_nt_k<BVB>(aKb[i], sU + 16 * R * LDB, LDB, sDS + 16 * cb * LDB, LDB);
        mma_nt_k<BVB>(aW[i], sDU + 16 * R * LDB, LDB, sS0 + 16 * cb * LDB, LDB);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NCT) {
        const int R = t / NB, I = t % NB;
        mma_nt_k<BVB>(aP[i], sDO + 16 * R * LDB, LDB, sU + 16 * I * LDB, LDB);
        mma_nt_k<BVB>(aT[i], sDU + 16 * R * LDB, LDB, sWV + 16 * I * LDB, LDB);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < SPASS; ++p) {
    float part = rs[p];
#pragma unroll
    for (int off = 1; off < ST4; off <<= 1) part += __shfl_xor(part, off);
    const int c = st_c + p * SROWS;
    if (st_j4 == 0 && c < DK) sEx[c] = part;
  }
  __syncthreads();

  // ---- phase A: dT, dKh, dA ----
  // running gradients at the lane's C x DK positions
  float gq[KPW][4], gk[KPW][4], gb[KPW][4];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool on = t < Cfg::NKT;
      const int r = 16 * R + 4 * lg + e;
      const float e1 = pe1[i][e];
      const float eg = on ? e1 * sCh[2 * DK + c] : 0.f;
      const float ec = on ? sCh[3 * DK + c] * __builtin_amdgcn_rcpf(e1) : 0.f;
      gq[i][e] = aQh[i][e] * eg;           // dQs exp(g)
      gk[i][e] = aKb[i][e] * ec;           // dKb exp(g_C - g)
      gb[i][e] = 0.f;
      aKb[i][e] = on ? pk[i][e] * ec * aKb[i][e] : 0.f;  // Kb * dKb for the exit term
      (void)r;
    }
    if (t < Cfg::NKT) store_tile(sDW + 16 * R * LDK + 16 * cb, LDK, aW[i], -1.f);
    if (t < Cfg::NKT) store_tile_t(sDWT + 16 * cb * LDC + 16 * R, LDC, aW[i], -1.f);
  }
  // colsum_r(Kb * dKb): reduce the lane's 4 rows, then the 4 row groups of the wave,
  // then (below, through LDS) the row blocks held by other waves
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    float s = aKb[i][0] + aKb[i][1] + aKb[i][2] + aKb[i][3];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    aKb[i][0] = s;
  }
  __syncthreads();
  // dT += dW Kh^T  -> dT (operand), and per-wave colsum partials
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NCT) {
      const int R = t / NB, I = t % NB;
      mma_nt_k<DK>(aT[i], sDW + 16 * R * LDK, LDK, sKh + 16 * I * LDK, LDK);
      store_tile(sDTm + 16 * R * LDC + 16 * I, LDC, aT[i]);
    }
  }
  // dKh = T^T dW, folded into db, dk
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
      f32x4 acc = zero4();
      mma_nt<OpT>(acc, sTT + 16 * R * LDC + 16 * R, LDC, sDWT + 16 * cb * LDC + 16 * R, LDC, C - 16 * R);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float eg = pe1[i][e] * sCh[2 * DK + c];
        gb[i][e] += acc[e] * pk[i][e] * eg;
        gk[i][e] += acc[e] * pb[i][e] * eg;
      }
    }
  }
  __syncthreads();
  // M = dT T^T -> M^T
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NCT) {
      const int R = t / NB, I = t % NB;
      f32x4 acc = zero4();
      mma_nt<OpT>(acc, sDTm + 16 * R * LDC, LDC, sTm + 16 * I * LDC, LDC, 16 * (I + 1));
      store_tile_t(sMT + 16 * I * LDC + 16 * R, LDC, acc);
    }
  }
  __syncthreads();
  // dA = strict_lower(-T^T M)
  f32x4 aA[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int t = wid + NW * i;
    aA[i] = zero4();
    if (t < Cfg::NCT) {
      const int R = t / NB, I = t % NB;
      if (I <= R) mma_nt<OpT>(aA[i], sTT + 16 * R * LDC + 16 * R, LDC, sMT + 16 * I * LDC + 16 * R, LDC, C - 16 * R);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
        aA[i][e] = row > col ? -aA[i][e] : 0.f;
        aP[i][e] = row >= col ? aP[i][e] : 0.f;
      }
    }
  }
  __syncthreads();  // every reader of the persistent buffers and of phase A is done

  // ---- phase B: products with the wide-range Gram factors ----
  constexpr int WP = Cfg::WPARTS;
  constexpr int KW = Cfg::kWM / (int)sizeof(WideT);                // elements per [C][LDC] part
  WideT* wdA = sW;                  // [WP][C][LDC]
  WideT* wdAT = sW + WP * KW;
  WideT* wdP = sW + 2 * WP * KW;
  WideT* wdPT = sW + 3 * WP * KW;
  auto put_wide = [&](WideT* base, int off, float x) {
    if constexpr (F32IN) base[off] = x;
    else st_split(base, base + KW, off, x);
  };
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NCT) {
      const int R = t / NB, I = t % NB;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
        put_wide(wdA, row * LDC + col, aA[i][e]);
        put_wide(wdAT, col * LDC + row, aA[i][e]);
        put_wide(wdP, row * LDC + col, aP[i][e]);
        put_wide(wdPT, col * LDC + row, aP[i][e]);
      }
    }
  }
  constexpr int KWF = DK * LDC;                                    // elements per factor part
  // factor^T [DK][LDC] from the lane's positions: which = 0: Kt', 1: Kh', 2: Qh'
  auto put_factor = [&](int which) {
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NKT) {
        const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          const float e1 = pe1[i][e];
          const float x = which == 0 ? pk[i][e] * __builtin_amdgcn_rcpf(e1)
                        : which == 1 ? pb[i][e] * pk[i][e] * e1 : pq[i][e] * e1;
          if constexpr (F32IN) sWF[c * LDC + r] = x;
          else st_split(sWF, sWF + KWF, c * LDC + r, x);
        }
      }
    }
  };
  auto wide_mma = [&](f32x4& acc, const WideT* X, int xoff, const WideT* Y, int yoff, int K) {
    if constexpr (F32IN) mma_nt<float>(acc, X + xoff, LDC, Y + yoff, LDC, K);
    else mma_nt_split(acc, X + xoff, X + KW + xoff, LDC, Y + yoff, Y + KWF + yoff, LDC, K);
  };
  put_factor(0);
  __syncthreads();
  // dKh' = dA Kt' ; dQh' = dP Kt'
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16;
      f32x4 x1 = zero4(), x2 = zero4();
      wide_mma(x1, wdA, 16 * R * LDC, sWF, 16 * cb * LDC, 16 * (R + 1));
      wide_mma(x2, wdP, 16 * R * LDC, sWF, 16 * cb * LDC, 16 * (R + 1));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float e1 = pe1[i][e];
        gb[i][e] += x1[e] * pk[i][e] * e1;
        gk[i][e] += x1[e] * pb[i][e] * e1;
        gq[i][e] += x2[e] * e1;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  put_factor(1);
  __syncthreads();
  // dKt' = dA^T Kh' + dP^T Qh'
  f32x4 aKt[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    aKt[i] = zero4();
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16;
      wide_mma(aKt[i], wdAT, 16 * R * LDC + 16 * R, sWF, 16 * cb * LDC + 16 * R, C - 16 * R);
    }
  }
  __syncthreads();
  put_factor(2);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16;
      wide_mma(aKt[i], wdPT, 16 * R * LDC + 16 * R, sWF, 16 * cb * LDC + 16 * R, C - 16 * R);
#pragma unroll
      for (int e = 0; e < 4; ++e) gk[i][e] += aKt[i][e] * __builtin_amdgcn_rcpf(pe1[i][e]);
    }
  }
  __syncthreads();  // phase B buffers are dead

  // ---- outputs dq, dk, db (staged through LDS for full-row stores); x = q dq + 2 b db - k dk ----
  // per-wave colsum partials of Kb * dKb (one wave per row block of each column block)
  for (int e = tid; e < NW * DK; e += NT) sExW[e] = 0.f;
  float* sOq = sX + C * DK;
  float* sOk = sX + 2 * C * DK;
  float* sOb = sX + 3 * C * DK;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    if (t < Cfg::NKT) {
      const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
      if (lg == 0) sExW[R * DK + c] = aKb[i][0];  // row block R of column c: a single writer
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        sX[r * DK + c] = pq[i][e] * gq[i][e] + 2.f * pb[i][e] * gb[i][e] - pk[i][e] * gk[i][e];
        if constexpr (Cfg::kStage) {
          sOq[r * DK + c] = gq[i][e];
          sOk[r * DK + c] = gk[i][e];
          sOb[r * DK + c] = gb[i][e];
        } else if (r < Lr) {  // no room to stage: column-per-lane stores
          const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
          a.dq[idx] = gq[i][e];
          a.dk[idx] = gk[i][e];
          a.db[idx] = gb[i][e];
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; Cfg::kStage && e < C * (DK / 4); e += NT) {
    const int r = e / (DK / 4), c4 = 4 * (e % (DK / 4));
    if (r < Lr) {
      const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c4;
      *reinterpret_cast<float4*>(a.dq + idx) = *reinterpret_cast<const float4*>(sOq + r * DK + c4);
      *reinterpret_cast<float4*>(a.dk + idx) = *reinterpret_cast<const float4*>(sOk + r * DK + c4);
      *reinterpret_cast<float4*>(a.db + idx) = *reinterpret_cast<const float4*>(sOb + r * DK + c4);
    }
  }
  // dlog_alpha: reverse cumulative sum over the chunk plus the exit term
  {
    constexpr int RPS = KS::LA_RPS, SEGS = KS::LA_SEGS;
    const int c = ks.la_c, sg = ks.la_sg;  // 4 channels c..c+3, rows sg*RPS ..
    float4 loc[RPS];
    if (ks.la_on) {
      float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = RPS - 1; i >= 0; --i) {
        const float4 x = *reinterpret_cast<const float4*>(sX + (sg * RPS + i) * DK + c);
        run.x += x.x; run.y += x.y; run.z += x.z; run.w += x.w;
        loc[i] = run;
      }
      *reinterpret_cast<float4*>(sTot + sg * DK + c) = run;
    }
    __syncthreads();
    if (ks.la_on) {
      float after[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < SEGS; ++s2) {
        if (s2 > sg) {
          const float4 tt = *reinterpret_cast<const float4*>(sTot + s2 * DK + c);
          after[0] += tt.x; after[1] += tt.y; after[2] += tt.z; after[3] += tt.w;
        }
      }
      float ex[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ex[j] = __expf(sCh[DK + c + j]) * sEx[c + j] + after[j];
#pragma unroll
        for (int R = 0; R < NB; ++R) ex[j] += sExW[R * DK + c + j];
      }
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
        const int r = sg * RPS + i;
        if (r < Lr)
          *reinterpret_cast<float4*>(a.dlog_alpha + baseK + (int64_t)(t0 + r) * rowK + c) =
              make_float4(loc[i].x + ex[0], loc[i].y + ex[1], loc[i].z + ex[2], loc[i].w + ex[3]);
      }
    }
  }
}

// =============================================================================
// dispatch
// =============================================================================
static int pick_bv_bwd(int B, int H, int Dv, bool f32) {
  const int maxbv = f32 ? 32 : 64;
  int bv = Dv < maxbv ? Dv : maxbv;
  while (bv > 16 && (long)B * H * (Dv / bv) < 256) bv /= 2;
  return bv;
}

template <int DK, int C, int BV, bool F32IN>
static hipError_t launch_dstate_t(const BwdArgs& a, hipStream_t s) {
  if constexpr (!DstCfg<DK, C, BV, F32IN>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int nv = a.Dv / BV, nbh = a.B * a.H;
    hipLaunchKernelGGL((gdn2_bwd_dstate_kernel<DK, C, BV, F32IN>), dim3(((nbh + 7) / 8) * 8 * nv),
                       dim3(kDstThreads), 0, s, a);
    return hipGetLastError();
  }
}

template <int DK, int C, int BVB, bool F32IN>
static hipError_t launch_grad_t(const BwdArgs& a, hipStream_t s) {
  if constexpr (!GradCfg<DK, C, BVB, F32IN>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int NC = (a.T + C - 1) / C;
    if (a.records)
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<DK, C, BVB, F32IN, true>), dim3(a.B * a.H * NC), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<DK, C, BVB, F32IN, false>), dim3(a.B * a.H * NC), dim3(512), 0, s, a);
    return hipGetLastError();
  }
}

// value tile of the gradient kernel's inner loop: 32 (16 for fp32 inputs), never wider than Dv
template <int DK, int C, bool F32IN>
static hipError_t launch_grad(const BwdArgs& a, hipStream_t s) {
  if (F32IN || a.Dv == 16) return launch_grad_t<DK, C, 16, F32IN>(a, s);
  if constexpr (F32IN) return hipErrorInvalidValue;
  else return launch_grad_t<DK, C, 32, F32IN>(a, s);
}

template <int DK, int C, bool F32IN>
static hipError_t launch_bwd_c(const BwdArgs& a, hipStream_t s) {
  hipError_t e;
  switch (pick_bv_bwd(a.B, a.H, a.Dv, F32IN)) {
    case 16: e = launch_dstate_t<DK, C, 16, F32IN>(a, s); break;
    case 32: e = launch_dstate_t<DK, C, 32, F32IN>(a, s); break;
    case 64:
      if constexpr (F32IN) e = hipErrorInvalidValue;
      else e = launch_dstate_t<DK, C, 64, F32IN>(a, s);
      break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_grad<DK, C, F32IN>(a, s);
}

template <int DK, bool F32IN>
static hipError_t launch_bwd_dk(const BwdArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_bwd_c<DK, 16, F32IN>(a, s);
    case 32: return launch_bwd_c<DK, 32, F32IN>(a, s);
    case 64: return launch_bwd_c<DK, 64, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_bwd_f(const BwdArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_bwd_dk<16, F32IN>(a, s);
    case 32: return launch_bwd_dk<32, F32IN>(a, s);
    case 64: return launch_bwd_dk<64, F32IN>(a, s);
    case 128: return launch_bwd_dk<128, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.f32_inputs ? launch_bwd_f<true>(a, stream) : launch_bwd_f<false>(a, stream);
}

template <int DK, bool F32IN>
static hipError_t launch_grad_dk(const BwdArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_grad<DK, 16, F32IN>(a, s);
    case 32: return launch_grad<DK, 32, F32IN>(a, s);
    case 64: return launch_grad<DK, 64, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_grad_f(const BwdArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_grad_dk<16, F32IN>(a, s);
    case 32: return launch_grad_dk<32, F32IN>(a, s);
    case 64: return launch_grad_dk<64, F32IN>(a, s);
    case 128: return launch_grad_dk<128, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream) {
  return a.f32_inputs ? launch_grad_f<true>(a, stream) : launch_grad_f<false>(a, stream);
}

template <int DK, int C, bool F32IN>
static bool bwd_fits() {
  return GradCfg<DK, C, 16, F32IN>::kFits && (F32IN || GradCfg<DK, C, 32, F32IN>::kFits) &&
         DstCfg<DK, C, 16, F32IN>::kFits && DstCfg<DK, C, 32, F32IN>::kFits &&
         (F32IN || DstCfg<DK, C, 64, F32IN>::kFits);
}

template <int DK, bool F32IN>
static bool grad_fits_c(int chunk) {
  switch (chunk) {
    case 16: return GradCfg<DK, 16, 16, F32IN>::kFits && (F32IN || GradCfg<DK, 16, 32, F32IN>::kFits);
    case 32: return GradCfg<DK, 32, 16, F32IN>::kFits && (F32IN || GradCfg<DK, 32, 32, F32IN>::kFits);
    case 64: return GradCfg<DK, 64, 16, F32IN>::kFits && (F32IN || GradCfg<DK, 64, 32, F32IN>::kFits);
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

template <int DK, bool F32IN>
static bool bwd_fits_c(int chunk) {
  switch (chunk) {
    case 16: return bwd_fits<DK, 16, F32IN>();
    case 32: return bwd_fits<DK, 32, F32IN>();
    case 64: return bwd_fits<DK, 64, F32IN>();
  }
  return false;
}

bool bwd_supported(int Dk, int Dv, int chunk, bool f32_inputs) {
  (void)Dv;
  switch (Dk) {
    case 16: return f32_inputs ? bwd_fits_c<16, true>(chunk) : bwd_fits_c<16, false>(chunk);
    case 32: return f32_inputs ? bwd_fits_c<32, true>(chunk) : bwd_fits_c<32, false>(chunk);
    case 64: return f32_inputs ? bwd_fits_c<64, true>(chunk) : bwd_fits_c<64, false>(chunk);
    case 128: return f32_inputs ? bwd_fits_c<128, true>(chunk) : bwd_fits_c<128, false>(chunk);
  }
  return false;
}

}  // namespace gdn2
