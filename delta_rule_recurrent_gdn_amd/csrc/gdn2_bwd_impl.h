// gdn2_bwd_impl.h -- gate-aware chunkwise backward of the Gated Delta Rule-2 operator: the
// per-chunk gradient kernels, instantiated per key width by gdn2_bwd_d*.hip.
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
// This file holds the chunk-parallel half: gdn2_bwd_grad_kernel, one workgroup
// per (batch, head, chunk), which takes the chunk's entry state (saved by the
// forward), the gradient of its exit state (from the reverse chain in
// gdn2_chain.hip) and T, P^T, Kh, Kb from the backward record (gdn2_prep.hip),
// and forms every per-token gradient of the chunk: a column phase (waves own
// value columns; U, dU and d(w v) as register chains), a key phase (waves own
// key-channel blocks; the contractions over the value axis), then dT, dA and
// the products with the wide-range Gram factors in LDS.
// Precision as in the forward: fp16 operands with fp32 accumulation, and a
// two-term bf16 split for the products with the wide-range factors Kh', Qh', Kt'.

#pragma once

#include "gdn2_chunk.h"
#include "gdn2_frag.h"
#include "gdn2_internal.h"
#include "gdn2_wide.h"

namespace gdn2 {

// =============================================================================
// chunk-parallel gradients
// =============================================================================

// Four input values kept in registers: fp32 as is, bf16 as their bits
// (exact: the inputs are bf16 numbers).
template <bool F32IN>
struct Vals4 {
  float v[4];
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
  // raw load of element idx (or of the always-valid safe when !ok); mask() zeroes it later
  __device__ __forceinline__ void set(int e, const void* base, int64_t idx, int64_t safe, bool ok) {
    v[e] = static_cast<const float*>(base)[ok ? idx : safe];
  }
  __device__ __forceinline__ void mask(int e, bool ok) { v[e] = ok ? v[e] : 0.f; }
  __device__ __forceinline__ float operator[](int e) const { return v[e]; }
};
template <>
struct Vals4<false> {
  uint32_t v[4];  // bf16 bits, one per register (no packing, so the loads need not wait for each other)
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0u; }
  __device__ __forceinline__ void set(int e, const void* base, int64_t idx, int64_t safe, bool ok) {
    v[e] = static_cast<const uint16_t*>(base)[ok ? idx : safe];
  }
  __device__ __forceinline__ void mask(int e, bool ok) { v[e] = ok ? v[e] : 0u; }
  __device__ __forceinline__ float operator[](int e) const { return __uint_as_float(v[e] << 16); }
};
template <int DK, int C, bool F32IN>
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
  static constexpr int LDC = KS::LDC, LDK = KS::LDK, LDCF = KS::LDCF;
  static constexpr int DVM = 128;                                  // widest value axis
  static constexpr int LDV = DVM + KS::PADOP;                      // rows over the value axis
  static constexpr int OPB = sizeof(OpT);
  static constexpr int WB = sizeof(WideT);
  // persistent (until the post-processing)
  static constexpr int oKh = 0;                                    // OpT [C][LDK]  b k exp(g)
  static constexpr int oKb = oKh + C * LDK * OPB;                  // OpT [C][LDK]  k exp(g_C - g)
  static constexpr int oTm = oKb + C * LDK * OPB;                  // OpT [C][LDC]  T
  static constexpr int oTT = oTm + C * LDC * OPB;                  // OpT [C][LDC]  T^T
  static constexpr int oPT = oTT + C * LDC * OPB;                  // OpT [C][LDC]  P^T
  static constexpr int oR = oPT + C * LDC * OPB;                   // phase region
  // phase G (gate cumsum)
  static constexpr int oG = oR;
  static constexpr int endPG = oG + KS::kGBytes;
  // phase V (U, dU and, for 16-bit operands, dO and w v over the whole value
  // axis: the row operands of the key-side contractions; fp32 operands read
  // dO and w v from global memory instead, to fit LDS)
  static constexpr bool kStageDO = !F32IN;
  static constexpr int oU = oR;                                    // OpT [C][LDV]
  static constexpr int oDU = oU + C * LDV * OPB;                   // OpT [C][LDV]
  static constexpr int oDO = oDU + C * LDV * OPB;                  // OpT [C][LDV]
  static constexpr int oWV = oDO + (kStageDO ? C * LDV * OPB : 0); // OpT [C][LDV]
  static constexpr int endV = oWV + (kStageDO ? C * LDV * OPB : 0);
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
    int m = endPG;
    if (endV > m) m = endV;
    if (endA > m) m = endA;
    if (endB > m) m = endB;
    return m;
  }();
  // cumsum segment totals: scratch of the gate cumsum and of the final scan
  // only, so they sit past the gate buffer and the output staging
  static constexpr int tot_at(int endD_) { return ((endPG > endD_ ? endPG : endD_) + 15) & ~15; }
  static constexpr int main_end(int endD_) {
    return endBase > tot_at(endD_) + KS::kTotBytes ? endBase : tot_at(endD_) + KS::kTotBytes;
  }
  static constexpr int kTail = KS::kChanBytes + 2 * DK * 4 + kWaves * DK * 4 + C * 8 * 4;
  static constexpr bool kStage = ((main_end(4 * C * DK * 4) + 15) & ~15) + kTail <= 160 * 1024;
  static constexpr int endD = (kStage ? 4 : 1) * C * DK * 4;
  static constexpr int oTOT = tot_at(endD);
  static constexpr int endMain = main_end(endD);
  // tail (always live)
  static constexpr int oCH = (endMain + 15) & ~15;
  static constexpr int oEX = oCH + KS::kChanBytes;                 // float [2][DK] exit-term pieces
  static constexpr int oEXW = oEX + 2 * DK * 4;                    // float [kWaves][DK] per-wave partials
  static constexpr int oRED = oEXW + kWaves * DK * 4;              // float [C][8] per-token partial sums
  static constexpr int kLdsBytes = oRED + C * 8 * 4;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;
  // the wide pass: block totals [NB][DK] and pair scales [npair][DK] over the per-wave partials,
  // which are live only in the output phase; phase B (from 0, below the tail) holds dA, dP
  // [C][LDCF], one factor [DK][LDCF], the block-relative cumulative log-decay and the running
  // gradient of b [C][DK + 4], all fp32
  static constexpr int oBS = oEXW;
  static constexpr int oPS = oBS + NB * DK * 4;
  static_assert((NB + wide_npair(NB)) * DK <= kWaves * DK, "block tables fit the per-wave partials");
  static constexpr int kWideB = (2 * C + DK) * LDCF * 4 + 2 * C * (DK + 4) * 4;

  static constexpr int NKT = NB * (DK / 16);                       // C x DK tiles
  static constexpr int KPW = (NKT + kWaves - 1) / kWaves;
  static constexpr int NCT = NB * NB;                              // C x C tiles
  static constexpr int CPW = (NCT + kWaves - 1) / kWaves;
};

// One (batch, head, chunk) item. T and P^T come from the backward records
// (a.records), the exit-state gradient from the reverse chain. WIDE = false:
// the fast path, whose results for chunks that carry the wide-decay flag in
// their record the WIDE = true pass then replaces (block-referenced decay
// factors, gdn2_wide.h).
// smem: GradCfg::kLdsBytes of LDS.
template <int DK, int C, bool F32IN, bool RAW, bool GS, bool S16, bool WIDE>
__device__ __forceinline__ void grad_chunk(const BwdArgs& a, int item, char* smem) {
  static_assert(!WIDE || GradCfg<DK, C, F32IN>::kWideB <= GradCfg<DK, C, F32IN>::oCH, "wide phase B fits");
  // GS: some gate holds one value per (token, head); the per-channel case compiles without that code
  const bool scalar_b = GS && a.scalar_b, scalar_w = GS && a.scalar_w, scalar_decay = GS && a.scalar_decay;
  using Cfg = GradCfg<DK, C, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  using WideT = typename Cfg::WideT;
  constexpr int NW = Cfg::kWaves, NB = Cfg::NB, NT = Cfg::kThreads;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDV = Cfg::LDV;
  constexpr int KPW = Cfg::KPW, CPW = Cfg::CPW;
  constexpr int KB16 = DK / 16;

  OpT* sKh = reinterpret_cast<OpT*>(smem + Cfg::oKh);
  OpT* sKb = reinterpret_cast<OpT*>(smem + Cfg::oKb);
  OpT* sTm = reinterpret_cast<OpT*>(smem + Cfg::oTm);
  OpT* sTT = reinterpret_cast<OpT*>(smem + Cfg::oTT);
  OpT* sPT = reinterpret_cast<OpT*>(smem + Cfg::oPT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  OpT* sU = reinterpret_cast<OpT*>(smem + Cfg::oU);
  OpT* sDU = reinterpret_cast<OpT*>(smem + Cfg::oDU);
  OpT* sDO = reinterpret_cast<OpT*>(smem + Cfg::oDO);
  OpT* sWV = reinterpret_cast<OpT*>(smem + Cfg::oWV);
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
  float* sRed = reinterpret_cast<float*>(smem + Cfg::oRED);  // scalar-gate gradients: [token][wave or block]

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int T = a.T, H = a.H, Dv = a.Dv;
  const int NC = (T + C - 1) / C;
  // (batch*head, chunk), chunk fastest; packed sequences: (head, global chunk)
  const ChunkLoc cl = chunk_loc(a.vl, T, H, DK, Dv, C, NC, item);
  if (cl.Lr <= 0) return;  // past the last chunk of a packed batch
  using Rec = Record<DK, C, F32IN, 1>;
  // (a chunk that the record pass flagged as wide-decay runs here as well, to no use: the wide pass
  // overwrites every gradient of it; checking the flag first would delay every workgroup's start)
  // 16-bit inputs: dO (and, through the reverse chain, dS) enter times a power of two (grad_scale);
  // every gradient is multiplied back by ginv before it is stored
  const float gsc = F32IN ? 1.f : grad_scale(a.gscale, cl.state), ginv = 1.f / gsc;
  const int t0 = cl.t0, Lr = cl.Lr;
  const int64_t rowK = (int64_t)H * DK, rowV = (int64_t)H * Dv;
  const int64_t baseK = cl.baseK, baseV = cl.baseV;
  const int64_t stOff = cl.item * DK * Dv;
  // chunk entry states: fp32, or fp16 (S16: the training pair's own copy, 16-bit inputs)
  using S0T = typename std::conditional<S16, _Float16, float>::type;
  static_assert(!S16 || !F32IN, "fp16 states go with 16-bit inputs");
  const S0T* S0g;
  if constexpr (S16) S0g = a.states16 + stOff;
  else S0g = a.chunk_states + stOff;
  // exit-state gradients: fp16 for 16-bit inputs (every use rounds them to fp16 operands anyway)
  using SdT = typename std::conditional<F32IN, float, _Float16>::type;
  const SdT* dSg = static_cast<const SdT*>(a.dS_chunks) + stOff;

  // ---- key-side preparation ----
  KS ks;
  ks.init(tid);
  ks.raw = RAW;
  ks.scalar_la = scalar_decay;
  // per-head scalar gates ([., T, H]): element offset of token 0 of this (batch row, head); the b and w
  // gates indexed as base + token * row + channel * stride in either layout
  const int64_t baseS = baseK / DK;
  const int64_t bBase = scalar_b ? baseS : baseK, bRow = scalar_b ? H : rowK;
  const int bCs = scalar_b ? 0 : 1;
  const int64_t wBase = scalar_w ? baseS : baseV, wRow = scalar_w ? H : rowV;
  const int wCs = scalar_w ? 0 : 1;
  // the column phase's gathers of dO, v and w (this wave's 16 value columns) are issued here as well,
  // ahead of the record units, so that one memory latency covers both
  using Fr = Frag<F32IN>;
  constexpr int KU = Fr::KU, UKd = Fr::units(DK), UCc = Fr::units(C), RC = C / 16;
  using RhsT = typename std::conditional<F32IN, f32x4, f16x8>::type;
  constexpr int NE = F32IN ? 4 : 8;
  using InT = typename std::conditional<F32IN, float, __bf16>::type;
  const int jc = 16 * wid + lr;
  float s0r[UKd][NE], dsr[UKd][NE];
  InT dor[UCc][NE], vr[RC][4], wr[RC][4];
  if (16 * wid < Dv) {
#pragma unroll
    for (int u = 0; u < UCc; ++u)
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int t = KU * u + Fr::kslot(lg, j);
        dor[u][j] = ld_sel(static_cast<const InT*>(a.dO), baseV + (int64_t)(t0 + t) * rowV + jc,
                           baseV + (int64_t)t0 * rowV + jc, t < Lr);
      }
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * R + 4 * lg + e;
        const int64_t idx = baseV + (int64_t)(t0 + t) * rowV + jc, safe = baseV + (int64_t)t0 * rowV + jc;
        vr[R][e] = ld_sel(static_cast<const InT*>(a.v), idx, safe, t < Lr);
        wr[R][e] = ld_sel(static_cast<const InT*>(a.w), wBase + (int64_t)(t0 + t) * wRow + jc * wCs,
                          wBase + (int64_t)t0 * wRow + jc * wCs, t < Lr);
      }
  }
  // T (and T^T) and P^T from the record's units; P^T units that lie wholly
  // below the diagonal are not stored (zero). The loads are issued before the gate cumsum, so that their
  // latency passes during it; they are unpacked after it
  using F = Frag<F32IN>;
  const char* rec = a.records + cl.item * Rec::kBytes;
  // units: T, P^T (chunk x chunk), then Kh, Kb (chunk x Dk); every load of
  // the wave first, then the unpacking
  constexpr int NU = Rec::RC * Rec::UC, NK = Rec::RC * Rec::UK, NUT = 2 * NU + 2 * NK;
  constexpr int UPW = (NUT + NW - 1) / NW;
  // (The unit index arithmetic is written out here: the same arithmetic in a
  // lambda with reference out-parameters, inside these unrolled loops,
  // compiled to code that unpacked wrong units for some sizes on gfx950.)
  uint4 uv[UPW];
  int uw[UPW], uR[UPW], uu[UPW];
#pragma unroll
  for (int p = 0; p < UPW; ++p) {
    const int t = wid + NW * p;
    const int which = t < NU ? 0 : t < 2 * NU ? 1 : t < 2 * NU + NK ? 2 : 3;
    const int tt = which == 0 ? t : which == 1 ? t - NU : which == 2 ? t - 2 * NU : t - 2 * NU - NK;
    const int nu = which < 2 ? Rec::UC : Rec::UK;
    const int ub = which == 0 ? Rec::u4 : which == 1 ? Rec::u0 : which == 2 ? Rec::u5 : Rec::u1;
    uw[p] = t < NUT ? which : -1;
    uR[p] = tt / nu;
    uu[p] = tt - uR[p] * nu;
    const int64_t off = t < NUT ? (int64_t)(ub + tt) * F::kUnitBytes : 0;  // past the units: any valid unit
    uv[p] = *reinterpret_cast<const uint4*>(rec + off + 16 * l);
  }
  ks.load_la(a.log_alpha, baseK, rowK, t0, Lr);
  ks.gates(sTot, sG, sCh);
  float* sBs = reinterpret_cast<float*>(smem + Cfg::oBS);
  float* sPS = reinterpret_cast<float*>(smem + Cfg::oPS);
  if constexpr (WIDE) {  // sG <- cumulative log-decay from each row's 16-token block start
    ks.load_la(a.log_alpha, baseK, rowK, t0, Lr);
    ks.gates_block(sTot, sG, sBs, sPS);
  }

  // the C x DK tiles this lane owns: rows 16R + 4lg + e, column 16cb + lr.
  // e1 = exp(g - g_m) there for the final chain rule (q, k and b are fetched
  // later, when the key phase starts, so that they are not live meanwhile);
  // the wide pass keeps the block-relative cumulative log-decay there instead.
  float pe1[KPW][4];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * R + 4 * lg + e;
      if constexpr (WIDE) pe1[i][e] = t < Cfg::NKT ? sG[r * DK + c] : 0.f;
      else pe1[i][e] = t < Cfg::NKT ? __expf(sG[r * DK + c] - sCh[c]) : 1.f;
    }
  }
  // exp(g) and exp(g_C - g) at a lane position from pe1 (row block R, channel c)
  auto eg_at = [&](float e1, int R, int c) -> float {
    if constexpr (WIDE) return __expf(wide_before<NB, DK>(sBs, R, c) + e1);
    else return e1 * sCh[2 * DK + c];
  };
  auto ec_at = [&](float e1, int R, int c) -> float {
    if constexpr (WIDE) return __expf((sBs[R * DK + c] - e1) + wide_after<NB, DK>(sBs, R, c));
    else return sCh[3 * DK + c] * __builtin_amdgcn_rcpf(e1);
  };
#pragma unroll
  for (int p = 0; p < UPW; ++p) {
    const int which = uw[p], R = uR[p], u = uu[p];
    // P^T units wholly below the diagonal are not stored: zero
    const bool zero = which == 1 && F::KU * u + F::KU - 1 < 16 * R;
    const uint4 v = zero ? make_uint4(0u, 0u, 0u, 0u) : uv[p];
    // (vector stores in the fp32-state kernel: 1.85 -> 1.83 ms for the B8 H16 T4096 separate backward;
    // in the fp16-state one they cost a spilled register and 5 us)
    constexpr bool VEC = !S16;
    if (which == 0) unpack_unit<F32IN, VEC>(v, R, u, C, sTm, LDC, sTT, LDC);
    else if (which == 1) unpack_unit<F32IN, VEC>(v, R, u, C, sPT, LDC, static_cast<OpT*>(nullptr), 0);
    else if (which >= 2)
      unpack_unit<F32IN, VEC>(v, R, u, DK, which == 2 ? sKh : sKb, LDK, static_cast<OpT*>(nullptr), 0);
  }

  // ---- column phase: each wave owns 16 value columns of the chunk ----
  // X = w v - Kh S0, U = T X, dU = P^T dO + Kb dS and d(w v) = T^T dU with
  // their right operands in registers: S0, dS and dO gathered straight into
  // operand slots, X and dU as the accumulators of the previous product
  // (lane layout of gdn2_frag.h); the left operands are row-major LDS rows
  // read in the same slot order. dw, dv leave from here; U and dU go to LDS
  // for the contractions over the value axis.
  __syncthreads();  // Kh, Kb, T, T^T, P^T are in LDS; the gate buffer is dead
  auto lds_unit = [&](const OpT* X, int ld, int row0, int k0, int K) -> uint4 {
    const OpT* p = X + (row0 + lr) * ld + k0 + 4 * lg;
    if constexpr (F32IN) {
      return *reinterpret_cast<const uint4*>(p);
    } else {
      const uint2 lo = *reinterpret_cast<const uint2*>(p);
      uint2 hi = make_uint2(0u, 0u);
      if (k0 + 16 < K) hi = *reinterpret_cast<const uint2*>(p + 16);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  // fp16 entry states (S16): the key phase's rows of S0 and dS (this wave's
  // key-channel block, 8 value columns per lane group and step) are fetched
  // as the column phase starts, so that they arrive during it instead of
  // opening the key phase with a wait (with per-head scalar gates too: B8 H16
  // T4096 KDA training step 2.43 -> 2.34 ms)
  constexpr bool kEarly = S16;
  constexpr int kNStepE = kEarly ? Cfg::DVM / 32 : 1;
  f16x8 eS[kNStepE], eD[kNStepE];
  auto fetch_rows = [&]() {
    if constexpr (kEarly) {
      const int d = 16 * (wid % KB16) + lr;
#pragma unroll
      for (int st = 0; st < kNStepE; ++st) {
        const int c0 = 32 * st + 8 * lg, cs = c0 < Dv ? c0 : 0;
        eS[st] = *reinterpret_cast<const f16x8*>(S0g + (int64_t)d * Dv + cs);
        eD[st] = *reinterpret_cast<const f16x8*>(dSg + (int64_t)d * Dv + cs);
      }
    }
  };
  if (16 * wid >= Dv) fetch_rows();  // a wave with no value columns
  if (16 * wid < Dv) {
    // S0 and dS in operand slots, then the key phase's rows of the same lines (read from L2)
#pragma unroll
    for (int u = 0; u < UKd; ++u)
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int d = KU * u + Fr::kslot(lg, j);
        s0r[u][j] = ld_sel(S0g, (int64_t)d * Dv + jc, jc, d < DK);
        dsr[u][j] = ld_sel(dSg, (int64_t)d * Dv + jc, jc, d < DK);
      }
    fetch_rows();
    __builtin_amdgcn_sched_barrier(0);
    RhsT s0f[UKd], dsf[UKd], dof[UCc];
    float vv[RC][4], ww[RC][4];
#pragma unroll
    for (int u = 0; u < UKd; ++u)
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        s0f[u][j] = static_cast<OpT>(s0r[u][j]);
        dsf[u][j] = static_cast<OpT>(dsr[u][j]);
      }
#pragma unroll
    for (int u = 0; u < UCc; ++u)
#pragma unroll
      for (int j = 0; j < NE; ++j) dof[u][j] = static_cast<OpT>(gsc * static_cast<float>(dor[u][j]));
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[R][e] = static_cast<float>(vr[R][e]);
        ww[R][e] = static_cast<float>(wr[R][e]);
      }
    if constexpr (RAW) {  // w = sigmoid(w_raw) on the sequence's rows (v is zero past it)
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int e = 0; e < 4; ++e) ww[R][e] = 16 * R + 4 * lg + e < Lr ? sigmoid_f(ww[R][e]) : 0.f;
    }
    // X = w v - Kh S0
    f32x4 X[RC];
#pragma unroll
    for (int R = 0; R < RC; ++R) {
      f32x4 acc = zero4();
#pragma unroll
      for (int u = 0; u < UKd; ++u) unit_mma(acc, lds_unit(sKh, LDK, 16 * R, KU * u, DK), s0f[u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) X[R][e] = vv[R][e] * ww[R][e] - acc[e];
    }
    // right operands over the chunk's tokens from accumulator tiles
    auto rhs_c = [&](const f32x4 (&Y)[RC], int u) -> RhsT {
      if constexpr (F32IN) return Y[u];
      else return rhs_from_acc(Y[2 * u], 2 * u + 1 < RC ? Y[2 * u + 1] : zero4());
    };
    // U = T X (T lower triangular: contraction units past the row block are zero)
    f32x4 Uc[RC], dU[RC];
#pragma unroll
    for (int R = 0; R < RC; ++R) {
      Uc[R] = zero4();
#pragma unroll
      for (int u = 0; u < UCc; ++u)
        if (KU * u <= 16 * R + 15) unit_mma(Uc[R], lds_unit(sTm, LDC, 16 * R, KU * u, C), rhs_c(X, u));
    }
    // dU = P^T dO + Kb dS (P^T upper triangular)
#pragma unroll
    for (int R = 0; R < RC; ++R) {
      dU[R] = zero4();
#pragma unroll
      for (int u = 0; u < UCc; ++u)
        if (KU * u + KU - 1 >= 16 * R) unit_mma(dU[R], lds_unit(sPT, LDC, 16 * R, KU * u, C), dof[u]);
#pragma unroll
      for (int u = 0; u < UKd; ++u) unit_mma(dU[R], lds_unit(sKb, LDK, 16 * R, KU * u, DK), dsf[u]);
    }
    // d(w v) = T^T dU -> dw, dv
#pragma unroll
    for (int R = 0; R < RC; ++R) {
      f32x4 acc = zero4();
#pragma unroll
      for (int u = 0; u < UCc; ++u)
        if (KU * u + KU - 1 >= 16 * R) unit_mma(acc, lds_unit(sTT, LDC, 16 * R, KU * u, C), rhs_c(dU, u));
      float gw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * R + 4 * lg + e;
        // pre-activation w: d/dw_raw = d/dw * w (1 - w)
        const float dwv = ginv * acc[e];
        gw[e] = t < Lr ? dwv * vv[R][e] * (RAW ? ww[R][e] * (1.f - ww[R][e]) : 1.f) : 0.f;
        if (t < Lr) {
          const int64_t idx = baseV + (int64_t)(t0 + t) * rowV + jc;
          // gradients are written once and never read here: non-temporal stores keep them from displacing
          // the lines the workgroups in flight still read (B8 H16 T4096 backward 1.48 -> 1.45 ms; the same
          // for the record pass's and the chains' stores made the training forward slower)
          if (!scalar_w) __builtin_nontemporal_store(gw[e], a.dw + idx);
          __builtin_nontemporal_store(dwv * ww[R][e], a.dv + idx);
        }
      }
      if (scalar_w) {  // per-head w: the sum over this wave's 16 columns, then over the waves (below)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = gw[e];
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          x += __shfl_xor(x, 8);
          if (lr == 0) sRed[(16 * R + 4 * lg + e) * 8 + wid] = x;
        }
      }
    }
    // U, dU, dO and w v row-major over the value axis
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * R + 4 * lg + e;
        sU[t * LDV + jc] = static_cast<OpT>(Uc[R][e]);
        sDU[t * LDV + jc] = static_cast<OpT>(dU[R][e]);
        if constexpr (Cfg::kStageDO) sWV[t * LDV + jc] = static_cast<OpT>(vv[R][e] * ww[R][e]);
      }
    if constexpr (Cfg::kStageDO) {
#pragma unroll
      for (int u = 0; u < UCc; ++u)
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          const int t = KU * u + Fr::kslot(lg, j);
          if (t < C) sDO[t * LDV + jc] = dof[u][j];
        }
    }
  }
  __syncthreads();
  if (scalar_w) {
    for (int t = tid; t < Lr; t += NT) {
      float x = 0.f;
      for (int w = 0; w < Dv / 16; ++w) x += sRed[t * 8 + w];
      a.dw[baseS + (int64_t)(t0 + t) * H] = x;
    }
  }

  // ---- key phase: contractions over the value axis ----
  //   dQs = dO S0^T, dKb = U dS^T, dU S0^T (C x DK);  dO U^T, dU (w v)^T (C x C)
  // Both operands are read row-major (S0 and dS from global memory; dO, U, dU
  // and w v from LDS), so the natural contraction order is used: 16-bit lane
  // group g takes 8 consecutive values at 8g (16x16x32), fp32 takes 4 at 4g
  // (four 16x16x4 products).
  f32x4 aQh[KPW], aKb[KPW], aW[KPW], aP[CPW], aT[CPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) aQh[i] = aKb[i] = aW[i] = zero4();
#pragma unroll
  for (int i = 0; i < CPW; ++i) aP[i] = aT[i] = zero4();
  // right operands: rows of S0 and dS of this wave's key-channel block, all
  // steps fetched at once; rowsum(S0 * dS) of those channels on the way
  constexpr int KV = F32IN ? 16 : 32;          // value columns per key-phase step
  constexpr int NV = F32IN ? 4 : 8;            // per lane group
  constexpr int NSTEP = Cfg::DVM / KV;
  using RhsT2 = typename std::conditional<F32IN, f32x4, f16x8>::type;
  const int cb0 = wid % KB16;                  // = t % KB16 for every tile t of this wave
  const bool rs_owner = wid < KB16;            // the wave whose first tile is in row block 0
  RhsT2 bS[NSTEP], bD[NSTEP];
  float rsum = 0.f;
  {
    const int d = 16 * cb0 + lr;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int c0 = KV * st + NV * lg;
      float xs[NV], xd[NV];
      const bool on = c0 < Dv;
      const int cs = on ? c0 : 0;  // unconditional loads, zeroed below
      const S0T* ps = S0g + (int64_t)d * Dv + cs;
      const SdT* pd = dSg + (int64_t)d * Dv + cs;
      if constexpr (kEarly) {  // fetched with the column phase's gathers
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          xs[j] = static_cast<float>(eS[st][j]);
          xd[j] = static_cast<float>(eD[st][j]);
        }
      } else if constexpr (S16) {  // NV = 8 halves: one 16-byte load
        const f16x8 h8 = *reinterpret_cast<const f16x8*>(ps);
#pragma unroll
        for (int j = 0; j < NV; ++j) xs[j] = static_cast<float>(h8[j]);
      }
#pragma unroll
      for (int j4 = 0; j4 < NV; j4 += 4) {
        if constexpr (!S16) {
          const float4 a4 = *reinterpret_cast<const float4*>(ps + j4);
          xs[j4] = a4.x; xs[j4 + 1] = a4.y; xs[j4 + 2] = a4.z; xs[j4 + 3] = a4.w;
        }
        if constexpr (F32IN) {
          const float4 b4 = *reinterpret_cast<const float4*>(pd + j4);
          xd[j4] = b4.x; xd[j4 + 1] = b4.y; xd[j4 + 2] = b4.z; xd[j4 + 3] = b4.w;
        }
      }
      if constexpr (!F32IN && !kEarly) {  // NV = 8 halves: one 16-byte load
        const f16x8 h8 = *reinterpret_cast<const f16x8*>(pd);
#pragma unroll
        for (int j = 0; j < NV; ++j) xd[j] = static_cast<float>(h8[j]);
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        xs[j] = on ? xs[j] : 0.f;
        xd[j] = on ? xd[j] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        bS[st][j] = static_cast<OpT>(xs[j]);
        bD[st][j] = static_cast<OpT>(xd[j]);
        rsum += xs[j] * xd[j];
      }
    }
  }
  // q, k, b at the lane's C x DK positions (for the chain rule after the key
  // phase): raw loads issued after the key-phase operands, so those arrive
  // first; zeroed past the sequence once the key phase is done
  Vals4<F32IN> pq[KPW], pk[KPW], pb[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
    const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * R + 4 * lg + e;
      const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
      const int64_t safe = baseK + (int64_t)t0 * rowK + (c < DK ? c : 0);  // row 0 of the chunk always exists
      const bool ok = t < Cfg::NKT && r < Lr;
      pq[i].set(e, a.q, idx, safe, ok);
      pk[i].set(e, a.k, idx, safe, ok);
      // b per channel, or one value per (token, head): base + token * row + channel * stride
      const int64_t ib = bBase + (int64_t)(t0 + r) * bRow + c * bCs, sb = bBase + (int64_t)t0 * bRow + (c < DK ? c : 0) * bCs;
      pb[i].set(e, a.b, ib, sb, ok);
    }
  }
  auto lds_rows = [&](const OpT* X, int row, int c0) -> RhsT2 {
    const RhsT2 r = *reinterpret_cast<const RhsT2*>(X + row * LDV + (c0 < Dv ? c0 : 0));
    return c0 < Dv ? r : RhsT2{};
  };
  // dO and w v rows (LDS when staged, else global memory; rows past the sequence are zero)
  auto do_rows = [&](int row, int c0) -> RhsT2 {
    if constexpr (Cfg::kStageDO) {
      return lds_rows(sDO, row, c0);
    } else {
      const bool on = row < Lr && c0 < Dv;
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.dO) + baseV +
                                                        (int64_t)(t0 + (on ? row : 0)) * rowV + (on ? c0 : 0));
      return on ? RhsT2{x.x, x.y, x.z, x.w} : RhsT2{};
    }
  };
  auto wv_rows = [&](int row, int c0) -> RhsT2 {
    if constexpr (Cfg::kStageDO) {
      return lds_rows(sWV, row, c0);
    } else {
      const bool on = row < Lr && c0 < Dv;
      const int64_t idx = baseV + (int64_t)(t0 + (on ? row : 0)) * rowV + (on ? c0 : 0);
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + idx);
      const float4 y0 = load_la4(static_cast<const float*>(a.w), idx, baseS + (int64_t)(t0 + (on ? row : 0)) * H,
                                 scalar_w);  // per-channel, or the token-head's value broadcast
      float4 y = y0;
      if constexpr (RAW) y = make_float4(sigmoid_f(y.x), sigmoid_f(y.y), sigmoid_f(y.z), sigmoid_f(y.w));
      return on ? RhsT2{x.x * y.x, x.y * y.y, x.z * y.z, x.w * y.w} : RhsT2{};
    }
  };
  auto kmma = [&](f32x4& acc, const RhsT2& x, const RhsT2& y) {
    if constexpr (F32IN) acc = unit_mma_ff(acc, x, y);
    else acc = mfma16x16x32(x, y, acc);
  };
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int c0 = KV * st + NV * lg;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NKT) {
        const int row = 16 * (t / KB16) + lr;
        const RhsT2 xo = do_rows(row, c0), xu = lds_rows(sU, row, c0), xdu = lds_rows(sDU, row, c0);
        kmma(aQh[i], xo, bS[st]);
        kmma(aW[i], xdu, bS[st]);
        kmma(aKb[i], xu, bD[st]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NCT) {
        const int row = 16 * (t / NB) + lr, col = 16 * (t % NB) + lr;
        kmma(aP[i], do_rows(row, c0), lds_rows(sU, col, c0));
        kmma(aT[i], lds_rows(sDU, row, c0), wv_rows(col, c0));
      }
    }
  }
  // b past the sequence is zero; pre-activation gates keep sigmoid(b_raw) as fp32 values in pbr
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int t = wid + NW * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = t < Cfg::NKT && 16 * (t / KB16) + 4 * lg + e < Lr;
      pq[i].mask(e, ok);
      pk[i].mask(e, ok);
      pb[i].mask(e, ok);
    }
  }
  float pbr[RAW ? KPW : 1][4];
  if constexpr (RAW) {
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = t < Cfg::NKT && 16 * (t / KB16) + 4 * lg + e < Lr;
        pbr[i][e] = ok ? sigmoid_f(pb[i][e]) : 0.f;
      }
    }
  }
  auto bval = [&](int i, int e) -> float {
    if constexpr (RAW) return pbr[i][e];
    else return pb[i][e];
  };
  rsum += __shfl_xor(rsum, 16);
  rsum += __shfl_xor(rsum, 32);
  if (rs_owner && lg == 0) sEx[16 * cb0 + lr] = ginv * rsum;
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
      const float eg = on ? eg_at(e1, on ? R : 0, c) : 0.f;
      const float ec = on ? ec_at(e1, on ? R : 0, c) : 0.f;
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
        const float eg = eg_at(pe1[i][e], R, c);
        gb[i][e] += acc[e] * pk[i][e] * eg;
        gk[i][e] += acc[e] * bval(i, e) * eg;
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

  if constexpr (WIDE) {
    // ---- phase B, wide-decay chunk: the products with the decay between tokens, exactly.
    // Blocks R > I through fp32 matrix cores, exp(g_r - g_i) = exp(gb_r) s_RI exp(Bs_I - gb_i)
    // (gdn2_wide.h); the diagonal blocks pair by pair. Register-light: the running gradients of
    // q and k wait in dq and dk (rows of the sequence), that of b in LDS; the inputs are read
    // again from global memory; q, k, b are reloaded into registers afterwards. ----
    constexpr int LDF = Cfg::LDCF;
    constexpr int LDD = DK + 4;
    float* wdA = reinterpret_cast<float*>(smem);  // [C][LDF] dA (strict lower)
    float* wdP = wdA + C * LDF;                   // [C][LDF] dP (lower incl.)
    float* wF = wdP + C * LDF;                    // [DK][LDF] one decayed factor, transposed
    float* wG = wF + DK * LDF;                    // [C][LDD] block-relative cumulative log-decay
    float* wB = wG + C * LDD;                     // [C][LDD] running gradient of b
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NCT) {
        const int R = t / NB, I = t % NB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
          wdA[row * LDF + col] = aA[i][e];
          wdP[row * LDF + col] = aP[i][e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NKT) {
        const int R = t / KB16, c = 16 * (t % KB16) + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          wG[r * LDD + c] = pe1[i][e];
          wB[r * LDD + c] = gb[i][e];
          if (r < Lr) {
            const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
            a.dq[idx] = gq[i][e];
            a.dk[idx] = gk[i][e];
          }
        }
      }
    }
    // q, k and the activated b at position (r, c), zero past the sequence
    auto in_at = [&](int r, int c, float& qv, float& kv, float& bv) {
      const bool ok = r < Lr;
      const int rr = t0 + (ok ? r : 0);
      const int64_t idx = baseK + (int64_t)rr * rowK + c;
      qv = ok ? load1<F32IN>(a.q, idx) : 0.f;
      kv = ok ? load1<F32IN>(a.k, idx) : 0.f;
      bv = ok ? load1<F32IN>(a.b, bBase + (int64_t)rr * bRow + c * bCs) : 0.f;
      if (RAW && ok) bv = sigmoid_f(bv);
    };
    auto add_out = [&](float* out, int r, int c, float x) {
      if (r < Lr) out[baseK + (int64_t)(t0 + r) * rowK + c] += x;
    };
    // factor^T over every position: 0: k exp(Bs_R - gb) (column factor), 1: b k exp(gb), 2: q exp(gb)
    auto put_wf = [&](int which) {
#pragma unroll 1
      for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, c = e - r * DK;
        float qv, kv, bv;
        in_at(r, c, qv, kv, bv);
        const float gbv = wG[r * LDD + c];
        wF[c * LDF + r] = which == 0 ? kv * __expf(sBs[(r >> 4) * DK + c] - gbv)
                                     : (which == 1 ? bv * kv : qv) * __expf(gbv);
      }
    };
    // acc += X Y^T over one 16-token block: X row lr at X[lr * ldx], token k at X[k * tx];
    // Y row lr (a channel of the factor) with its tokens contiguous
    auto blk_mma = [&](f32x4& acc, const float* X, int ldx, int tx, const float* Y) {
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) acc = mfma16x16x4(X[lr * ldx + (k0 + lg) * tx], Y[lr * LDF + k0 + lg], acc);
    };
    __syncthreads();
    put_wf(0);
    __syncthreads();
    // rows of block R against the columns of earlier blocks: the dKh' and dQh' parts
#pragma unroll 1
    for (int t = wid; t < Cfg::NKT; t += NW) {
      const int R = t / KB16, cb = t % KB16, c = 16 * cb + lr;
      f32x4 x1 = zero4(), x2 = zero4();
#pragma unroll 1
      for (int I = 0; I < R; ++I) {
        f32x4 a1 = zero4(), a2 = zero4();
        blk_mma(a1, wdA + 16 * R * LDF + 16 * I, LDF, 1, wF + 16 * cb * LDF + 16 * I);
        blk_mma(a2, wdP + 16 * R * LDF + 16 * I, LDF, 1, wF + 16 * cb * LDF + 16 * I);
        const float sc = I + 2 <= R ? sPS[wide_pair(R, I) * DK + c] : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x1[e] += sc * a1[e];
          x2[e] += sc * a2[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        float qv, kv, bv;
        in_at(r, c, qv, kv, bv);
        const float E = __expf(wG[r * LDD + c]);
        wB[r * LDD + c] += x1[e] * kv * E;
        add_out(a.dk, r, c, x1[e] * bv * E);
        add_out(a.dq, r, c, x2[e] * E);
      }
    }
    __syncthreads();
    // columns of block I against the rows of later blocks: dKt' = dA^T Kh' + dP^T Qh'
#pragma unroll 1
    for (int pass = 1; pass <= 2; ++pass) {
      put_wf(pass);
      __syncthreads();
      const float* M = pass == 1 ? wdA : wdP;
#pragma unroll 1
      for (int t = wid; t < Cfg::NKT; t += NW) {
        const int I = t / KB16, cb = t % KB16, c = 16 * cb + lr;
        f32x4 x = zero4();
#pragma unroll 1
        for (int R = I + 1; R < NB; ++R) {
          f32x4 a1 = zero4();
          blk_mma(a1, M + 16 * R * LDF + 16 * I, 1, LDF, wF + 16 * cb * LDF + 16 * R);
          const float sc = I + 2 <= R ? sPS[wide_pair(R, I) * DK + c] : 1.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] += sc * a1[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * lg + e;
          add_out(a.dk, r, c, x[e] * __expf(sBs[I * DK + c] - wG[r * LDD + c]));
        }
      }
      __syncthreads();
    }
    // the diagonal blocks, pair by pair: position (r, c) collects its row's terms (i <= r) and
    // its column's terms (rows i >= r) of its own 16-token block
#pragma unroll 1
    for (int t = wid; t < Cfg::NKT; t += NW) {
      const int R = t / KB16, c = 16 * (t % KB16) + lr;
#pragma unroll 1
      for (int e = 0; e < 4; ++e) {
        const int rl = 4 * lg + e, r = 16 * R + rl;
        float qr, kr, br;
        in_at(r, c, qr, kr, br);
        const float gr = wG[r * LDD + c];
        float dX = 0.f, dQh = 0.f, dY = 0.f;
#pragma unroll 1
        for (int il = 0; il < 16; ++il) {
          const int i = 16 * R + il;
          float qi, ki, bi;
          in_at(i, c, qi, ki, bi);
          const float gi = wG[i * LDD + c];
          if (il <= rl) {  // row r: dA_r,i k_i and dP_r,i k_i
            const float tt = ki * __expf(gr - gi);
            dX += (il < rl ? wdA[r * LDF + i] : 0.f) * tt;
            dQh += wdP[r * LDF + i] * tt;
          }
          if (il >= rl) {  // column r: dA_i,r (b k)_i and dP_i,r q_i
            dY += ((il > rl ? wdA[i * LDF + r] * bi * ki : 0.f) + wdP[i * LDF + r] * qi) * __expf(gi - gr);
          }
        }
        wB[r * LDD + c] += dX * kr;
        add_out(a.dk, r, c, dX * br + dY);
        add_out(a.dq, r, c, dQh);
      }
    }
    __syncthreads();
    // back into registers: the running gradients, and q, k, b at the lane's positions
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int t = wid + NW * i;
      const int R = t / KB16, c = 16 * (t % KB16) + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        const bool on = t < Cfg::NKT, ok = on && r < Lr;
        const int64_t idx = baseK + (int64_t)(t0 + (ok ? r : 0)) * rowK + (on ? c : 0);
        const int64_t safe = baseK + (int64_t)t0 * rowK;
        gq[i][e] = ok ? a.dq[idx] : 0.f;
        gk[i][e] = ok ? a.dk[idx] : 0.f;
        gb[i][e] = on ? wB[r * LDD + c] : 0.f;
        pq[i].set(e, a.q, idx, safe, ok);
        pk[i].set(e, a.k, idx, safe, ok);
        pb[i].set(e, a.b, bBase + (int64_t)(t0 + (ok ? r : 0)) * bRow + (on ? c : 0) * bCs, bBase + (int64_t)t0 * bRow,
                  ok);
        pq[i].mask(e, ok);
        pk[i].mask(e, ok);
        pb[i].mask(e, ok);
        if constexpr (RAW) pbr[i][e] = ok ? sigmoid_f(pb[i][e]) : 0.f;
      }
    }
    __syncthreads();
  } else {
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
                          : which == 1 ? bval(i, e) * pk[i][e] * e1 : pq[i][e] * e1;
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
          gk[i][e] += x1[e] * bval(i, e) * e1;
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
  }
  if constexpr (!F32IN) {  // the gradients without the upstream scale from here on
#pragma unroll
    for (int i = 0; i < KPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gq[i][e] *= ginv;
        gk[i][e] *= ginv;
        gb[i][e] *= ginv;
      }
  }

  // ---- outputs dq, dk, db (staged through LDS for full-row stores); x = q dq + 2 b db - k dk ----
  // pre-activation decay: sigmoid(a_raw) scales the decay gradient at its stores (the thread's rows of
  // the final scan); fetched here so that the loads are in flight during the output staging
  float4 araw[KS::LA_RPS];
  if (RAW && ks.la_on) {
#pragma unroll
    for (int i = 0; i < KS::LA_RPS; ++i) {
      const int r = ks.la_sg * KS::LA_RPS + i;
      const int rr = t0 + (r < Lr ? r : 0);
      araw[i] = load_la4(a.log_alpha, baseK + (int64_t)rr * rowK + ks.la_c, baseS + (int64_t)rr * H, scalar_decay);
    }
  }
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
      if (lg == 0) sExW[R * DK + c] = ginv * aKb[i][0];  // row block R of column c: a single writer
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        sX[r * DK + c] = pq[i][e] * gq[i][e] + 2.f * bval(i, e) * gb[i][e] - pk[i][e] * gk[i][e];
        // pre-activation b: d/db_raw = d/db * b (1 - b)
        if constexpr (RAW) gb[i][e] *= bval(i, e) * (1.f - bval(i, e));
        if constexpr (Cfg::kStage) {
          sOq[r * DK + c] = gq[i][e];
          sOk[r * DK + c] = gk[i][e];
          sOb[r * DK + c] = gb[i][e];
        } else if (r < Lr) {  // no room to stage: column-per-lane stores
          const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
          a.dq[idx] = gq[i][e];
          a.dk[idx] = gk[i][e];
          if (!scalar_b) a.db[idx] = gb[i][e];
        }
      }
      if (!Cfg::kStage && scalar_b) {  // per-head b, unstaged: sum over the tile's 16 channels, then the blocks
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = gb[i][e];
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          x += __shfl_xor(x, 8);
          if (lr == 0) sRed[(16 * R + 4 * lg + e) * 8 + cb] = x;
        }
      }
    }
  }
  __syncthreads();
  if (scalar_b) {
    if constexpr (Cfg::kStage) {
      // per-head b: row sums of the staged gradient, BP threads per row (DK / BP channels each)
      constexpr int BP = DK / 4 < 8 ? DK / 4 : 8, BCH = DK / BP;
      for (int e = tid; e < C * BP; e += NT) {  // groups of BP lanes are wholly in or out
        const int r = e / BP, part = e - r * BP;
        float x = 0.f;
#pragma unroll
        for (int c = part * BCH; c < (part + 1) * BCH; c += 4) {
          const float4 y = *reinterpret_cast<const float4*>(sOb + r * DK + c);
          x += (y.x + y.y) + (y.z + y.w);
        }
#pragma unroll
        for (int m = 1; m < BP; m *= 2) x += __shfl_xor(x, m);
        if (part == 0 && r < Lr) a.db[baseS + (int64_t)(t0 + r) * H] = x;
      }
    } else {
      for (int t = tid; t < Lr; t += NT) {
        float x = 0.f;
        for (int cb = 0; cb < KB16; ++cb) x += sRed[t * 8 + cb];
        a.db[baseS + (int64_t)(t0 + t) * H] = x;
      }
    }
  }
  for (int e = tid; Cfg::kStage && e < C * (DK / 4); e += NT) {
    const int r = e / (DK / 4), c4 = 4 * (e % (DK / 4));
    if (r < Lr) {
      const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c4;
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sOq + r * DK + c4), reinterpret_cast<f32x4*>(a.dq + idx));
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sOk + r * DK + c4), reinterpret_cast<f32x4*>(a.dk + idx));
      if (!scalar_b)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sOb + r * DK + c4), reinterpret_cast<f32x4*>(a.db + idx));
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
        const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
        float4 d = make_float4(loc[i].x + ex[0], loc[i].y + ex[1], loc[i].z + ex[2], loc[i].w + ex[3]);
        if constexpr (RAW) {
          // log_alpha = -softplus(a_raw): d/da_raw = d/dlog_alpha * (-sigmoid(a_raw))
          const float4 ar = araw[i];
          d = make_float4(-d.x * sigmoid_f(ar.x), -d.y * sigmoid_f(ar.y), -d.z * sigmoid_f(ar.z),
                          -d.w * sigmoid_f(ar.w));
        }
        if (!scalar_decay) {
          if (r < Lr) {
            const f32x4 dv4 = {d.x, d.y, d.z, d.w};
            __builtin_nontemporal_store(dv4, reinterpret_cast<f32x4*>(a.dlog_alpha + idx));
          }
        } else {
          // per-head decay: the sum over the row's channels, held by DK / 4 consecutive threads
          float x = d.x + d.y + d.z + d.w;
#pragma unroll
          for (int m = 1; m < DK / 4; m *= 2) x += __shfl_xor(x, m);
          if (c == 0 && r < Lr) a.dlog_alpha[baseS + (int64_t)(t0 + r) * H] = x;
        }
      }
    }
  }
}

// =============================================================================
// dispatch
// =============================================================================
// The per-chunk gradient pass: one workgroup per chunk (fast path).
template <int DK, int C, bool F32IN, bool RAW, bool GS, bool S16>
__global__ __launch_bounds__(512) void gdn2_bwd_grad_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GradCfg<DK, C, F32IN>::kLdsBytes];
  grad_chunk<DK, C, F32IN, RAW, GS, S16, false>(a, chunk_item_of_block(a.vl, a.T, a.H, C, blockIdx.x), smem);
}

// One wide-pass item as a called function, so that its register allocation does
// not carry the item loop of the kernel below.
template <int DK, int C, bool F32IN, bool RAW, bool GS, bool S16>
__device__ __attribute__((noinline)) void grad_chunk_wide(const BwdArgs& a, int item, char* smem) {
  grad_chunk<DK, C, F32IN, RAW, GS, S16, true>(a, item, smem);
}

// The chunks whose backward record carries the wide-decay flag, recomputed
// with the block-referenced decay factors. Workgroup w covers items w,
// w + gridDim.x, ...: their flags are read in parallel, the flagged items
// listed in LDS and processed one after another.
template <int DK, int C, bool F32IN, bool RAW, bool GS, bool S16>
__global__ __launch_bounds__(512) void gdn2_bwd_grad_wide_kernel(BwdArgs a, int nitems) {
  using Rec = Record<DK, C, F32IN, 1>;
  __shared__ __attribute__((aligned(16))) char smem[GradCfg<DK, C, F32IN>::kLdsBytes];
  __shared__ int list[kWideBatch];
  __shared__ int count;
  const int per = (nitems + (int)gridDim.x - 1) / (int)gridDim.x;
  for (int k0 = 0; k0 < per; k0 += kWideBatch) {
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    const int k = k0 + (int)threadIdx.x;
    const int64_t item = blockIdx.x + (int64_t)k * gridDim.x;
    if (threadIdx.x < kWideBatch && k < per && item < nitems) {
      const int f = *reinterpret_cast<const int*>(a.records + item * Rec::kBytes + wide_flag_offset<Rec>());
      if (f == 1) list[atomicAdd(&count, 1)] = (int)item;
    }
    __syncthreads();
    const int n = count;
    for (int j = 0; j < n; ++j) {
      grad_chunk_wide<DK, C, F32IN, RAW, GS, S16>(a, list[j], smem);
      __syncthreads();
    }
    __syncthreads();
  }
}

template <int DK, int C, bool F32IN, bool RAW, bool GS, bool S16>
static hipError_t launch_grad_pair(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = chunk_items(a.vl, a.B, a.T, a.H, C);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gdn2_bwd_grad_kernel<DK, C, F32IN, RAW, GS, S16>), dim3((unsigned)grid), dim3(512), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int wgrid = grid < kWideGrid ? (int)grid : kWideGrid;
  hipLaunchKernelGGL((gdn2_bwd_grad_wide_kernel<DK, C, F32IN, RAW, GS, S16>), dim3((unsigned)wgrid), dim3(512), 0, s,
                     a, (int)grid);
  return hipGetLastError();
}

template <int DK, int C, bool F32IN>
static hipError_t launch_grad_t(const BwdArgs& a, hipStream_t s) {
  if constexpr (!GradCfg<DK, C, F32IN>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    if (a.records == nullptr) return hipErrorInvalidValue;
    const bool gs = a.scalar_b || a.scalar_w || a.scalar_decay;
    if (a.states16 != nullptr) {
      if constexpr (F32IN) {
        return hipErrorInvalidValue;  // fp16 states go with 16-bit inputs
      } else {
        if (a.raw_gates && gs) return launch_grad_pair<DK, C, F32IN, true, true, true>(a, s);
        if (a.raw_gates) return launch_grad_pair<DK, C, F32IN, true, false, true>(a, s);
        if (gs) return launch_grad_pair<DK, C, F32IN, false, true, true>(a, s);
        return launch_grad_pair<DK, C, F32IN, false, false, true>(a, s);
      }
    }
    if (a.chunk_states == nullptr) return hipErrorInvalidValue;
    if (a.raw_gates && gs) return launch_grad_pair<DK, C, F32IN, true, true, false>(a, s);
    if (a.raw_gates) return launch_grad_pair<DK, C, F32IN, true, false, false>(a, s);
    if (gs) return launch_grad_pair<DK, C, F32IN, false, true, false>(a, s);
    return launch_grad_pair<DK, C, F32IN, false, false, false>(a, s);
  }
}

template <int DK, bool F32IN>
static hipError_t launch_grad_dk(const BwdArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_grad_t<DK, 16, F32IN>(a, s);
    case 32: return launch_grad_t<DK, 32, F32IN>(a, s);
    case 64: return launch_grad_t<DK, 64, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn2
