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
// gdn2_frag.h) and Ut as accumulator tiles: tile (R, jb) of 16 x 16 at
// element offset 256 * (R * Dv/16 + jb), lane l's 4 values (rows 4(l/16)+i,
// column l%16) contiguous, so the chain reads each tile with one load per lane;
// fp32 for fp32 inputs, fp16 for 16-bit inputs (U = Ut - W S becomes an fp16
// operand in each of its uses, so the stored Ut needs no more).
//
// Precision as in the single-pass forward: A and P from a two-term bf16 split
// of their decay-scaled factors (referenced to the chunk middle so that the
// exp(+-g) factors stay in range), all other operands fp16 for bf16 inputs;
// fp32 matrix cores for fp32 inputs.
//
// Layout for occupancy (two workgroups per CU at d_k = 128, chunk 64, bf16):
// each thread owns one row and 4 channels of every channel slice, so the
// in-chunk cumsum of log_alpha runs in registers (wave shuffles, then one
// cross-wave total); decayed q and the causal term (computed transposed, as
// P^T tiles, whose accumulators are P's record units) go straight to the
// workspace; the transposed decayed k and b*k share one LDS buffer in turn.

#include "gdn2_chunk.h"
#include "gdn2_frag.h"
#include "gdn2_internal.h"
#include "gdn2_wide.h"

namespace gdn2 {

// DIR 0: forward record (+ T (w v)); DIR 1: backward record (no value side);
// DIR 2: both records and T (w v) from one pass (the training forward).
template <int DK, int C, bool F32IN, int DIR>
struct PrepCfg {
  static constexpr int NT = 512, NW = NT / kWave;
  using KS = KSide<DK, C, F32IN, NT>;  // slice geometry and the blocked inversion
  using OpT = typename KS::OpT;
  using Rec = Record<DK, C, F32IN, DIR == 1 ? 1 : 0>;  // the record `rec` points at
  using RecB = Record<DK, C, F32IN, 1>;                // the backward record (DIR 1, 2)
  using F = Frag<F32IN>;
  static constexpr int NB = KS::NB, SW = KS::SW, NSL = KS::NSL;
  static constexpr int LDC = KS::LDC, LDCF = KS::LDCF, LDSW = KS::LDSW;
  static constexpr int OPB = sizeof(OpT);
  static constexpr int DVM = DIR != 1 ? 128 : 0;  // largest value width staged
  // thread -> (row, 4 channels of every slice): TPR threads per row
  static constexpr int TPR = SW / 4;
  static constexpr int RPW = kWave / TPR;        // rows per wave
  // Gram tiles: the strict-lower A tiles, then the causal term's tiles in the
  // orientation of each record written (DIR 2: both, half again as many)
  static constexpr int NGT = KS::NGT, NGT2 = DIR == 2 ? NGT + NGT / 2 : NGT, GPW = (NGT2 + NW - 1) / NW;
  // LDS
  static constexpr int oCH = 0;                                    // float [4][DK] g_m, g_C, exp(g_m), exp(g_C-g_m)
  static constexpr int oTOT = oCH + 4 * DK * 4;                    // float [NW][DK] per-wave cumsum totals
  static constexpr int oR = oTOT + NW * DK * 4;
  static constexpr int oSL = oR;                                   // Gram factor slices (factor phase)
  static constexpr int oAf = oR;                                   // float [C][LDCF] A, then T (after the Gram)
  static constexpr int oXs = oAf + KS::kAfBytes;
  // wide-decay chunks: per slice, three fp32 factors [C][LDW], then k and the block-relative
  // cumulative decay [C][LDW] with the diagonal-block tables [C][16] of A and P
  static constexpr int LDW = SW + 4;
  static constexpr int kWideFac = 3 * C * LDW * 4;
  static constexpr int kWideDiag = 2 * C * LDW * 4 + 2 * C * 16 * 4;
  static constexpr int kSlR = KS::kSlicesBytes > kWideFac ? (KS::kSlicesBytes > kWideDiag ? KS::kSlicesBytes : kWideDiag)
                                                          : (kWideFac > kWideDiag ? kWideFac : kWideDiag);
  static constexpr int endR = (kSlR > KS::kAfBytes + KS::kXsBytes ? kSlR : KS::kAfBytes + KS::kXsBytes);
  static constexpr int oT1 = oR + ((endR + 15) & ~15);            // OpT [DK][LDC]: Kb^T, later Kh^T
  static constexpr int oWVT = oT1 + DK * LDC * OPB;                // OpT [DVM][LDC] (w v)^T
  // (w v)^T row j holds its 8-token blocks permuted, block b at b ^ ((j / 8) & kWvSwz): the staging
  // writes of one wave cover 16 rows 8 apart, which would otherwise all start in the same LDS bank
  // (16-way conflicts; 2-way with the permutation). 16-bit operands only.
  static constexpr int kWvSwz = F32IN ? 0 : C / 8 - 1;
  static constexpr int oBS = oWVT + DVM * LDC * OPB;               // float [NB][DK] block totals (wide path)
  static constexpr int oPS = oBS + NB * DK * 4;                    // float [npair][DK] pair scales (wide path)
  static constexpr int kLdsBytes = oPS + wide_npair(NB) * DK * 4;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;
  static constexpr int VW_PT = (C * DVM / 8 + NT - 1) / NT;
};

// Byte offset, inside a record matrix with `nu` units per row tile, of the
// 4 consecutive contraction indices k0..k0+3 (k0 % 4 == 0) of row r.
template <bool F32IN>
__device__ __forceinline__ int unit_off4(int r, int k0, int nu) {
  using F = Frag<F32IN>;
  const int u = k0 / F::KU, kl = k0 - u * F::KU;
  const int g = (kl & 15) >> 2, half = F32IN ? 0 : (kl >> 4);
  return ((r >> 4) * nu + u) * F::kUnitBytes + 16 * ((r & 15) + 16 * g) + 8 * half;
}

// Gram tile t: kind 0 = a strict-lower tile of A, 1 = a causal-term tile computed
// as P^T (its accumulators are the forward record's P units), 2 = one computed as
// P (the backward record's P^T units); (R, I) its block in the lower triangle.
template <int DIR, int NGT>
__device__ __forceinline__ int gram_tile(int t, int& R, int& I) {
  constexpr int HALF = NGT / 2;
  const int kind = t < HALF ? 0 : (DIR == 0 ? 1 : (DIR == 1 ? 2 : (t < NGT ? 1 : 2)));
  tri_index(t < HALF ? t : (t < NGT ? t - HALF : t - NGT), R, I);
  return kind;
}

// One chunk (item) of the chunk-parallel record pass. WIDE = false: the fast path, which only
// flags a wide-decay chunk (and leaves its record to the WIDE = true pass); WIDE = true: the
// block-referenced factors of gdn2_wide.h, exact for any decay. smem: Cfg::kLdsBytes of LDS.
template <int DK, int C, bool F32IN, int DIR, bool WIDE>
__device__ __forceinline__ void prep_chunk(const FwdArgs& a, char* rec_base, float* ut_base, char* brec_base,
                                           int item, char* smem) {
  using Cfg = PrepCfg<DK, C, F32IN, DIR>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  using Rec = typename Cfg::Rec;
  using RecB = typename Cfg::RecB;
  using F = Frag<F32IN>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, SW = Cfg::SW, NSL = Cfg::NSL, TPR = Cfg::TPR;
  constexpr int LDC = Cfg::LDC, LDCF = Cfg::LDCF, LDSW = Cfg::LDSW;
  constexpr int NGT = Cfg::NGT, NGT2 = Cfg::NGT2, GPW = Cfg::GPW;

  float* sCh = reinterpret_cast<float*>(smem + Cfg::oCH);
  float* sTot = reinterpret_cast<float*>(smem + Cfg::oTOT);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);
  OpT* sT1 = reinterpret_cast<OpT*>(smem + Cfg::oT1);
  OpT* sWVT = reinterpret_cast<OpT*>(smem + Cfg::oWVT);

  // the wave index in a scalar register: per-wave branches and offsets stay scalar (B8 H16 T4096 single-pass
  // forward 1.34 -> 1.24 ms, training forward 0.86 -> 0.84 ms)
  const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid & (kWave - 1);

  const int Dv = a.Dv, T = a.T, H = a.H;
  const int NC = (T + C - 1) / C;
  // (batch*head, chunk), chunk fastest; packed sequences: (head, global chunk)
  const ChunkLoc cl = chunk_loc(a.vl, T, H, DK, Dv, C, NC, item);
  if (cl.Lr <= 0) return;  // past the last chunk of a packed batch
  const int t0 = cl.t0, Lr = cl.Lr;
  const int64_t rowK = (int64_t)H * DK, rowV = (int64_t)H * Dv;
  const int64_t baseK = cl.baseK, baseV = cl.baseV;
  char* rec = rec_base + cl.item * Rec::kBytes;  // forward record (DIR 0, 2), backward record (DIR 1)
  char* recB = DIR == 1 ? rec : (DIR == 2 ? brec_base + cl.item * RecB::kBytes : nullptr);
  // Ut: fp32 tiles for fp32 inputs, fp16 for 16-bit ones (each use of U = Ut - W S is an fp16 operand)
  char* ut = reinterpret_cast<char*>(ut_base) + cl.item * C * Dv * (F32IN ? 4 : 2);

  // ---- loads: row r, channels sl*SW + 4*c4 .. +3 of every slice sl ----
  const int r = tid / TPR, c4 = tid - r * TPR;
  const bool live = r < C;  // a row of the chunk (rows >= Lr are zero padding)
  Raw4<F32IN> rq[NSL], rk[NSL], rb[NSL];
  float g[NSL][4];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const int c0 = sl * SW + 4 * c4;
    if (live && r < Lr) {
      const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c0;
      const int64_t sidx = baseK / DK + (int64_t)(t0 + r) * H;  // per-head scalar gates: [., T, H]
      ld_raw(rq[sl], a.q, idx);
      ld_raw(rk[sl], a.k, idx);
      ld_raw_gate(rb[sl], a.b, idx, sidx, a.scalar_b);
      const float4 x = load_la4(a.log_alpha, idx, sidx, a.scalar_decay);
      g[sl][0] = x.x; g[sl][1] = x.y; g[sl][2] = x.z; g[sl][3] = x.w;
    } else {
      zero_raw(rq[sl]);
      zero_raw(rk[sl]);
      zero_raw(rb[sl]);
      g[sl][0] = g[sl][1] = g[sl][2] = g[sl][3] = 0.f;
    }
  }
  // (w v)^T for the whole value width, into its own LDS region
  if constexpr (DIR != 1) {
    const int vpr = Dv / 8;
#pragma unroll
    for (int i = 0; i < Cfg::VW_PT; ++i) {
      const int e = tid + NT * i, rr = e / vpr, j8 = e - rr * vpr;
      if (rr < C) {
        float vv[8], ww[8];
        if (rr < Lr) {
          const int64_t idx = baseV + (int64_t)(t0 + rr) * rowV + 8 * j8;
          load8<F32IN>(a.v, idx, vv);
          load8_gate<F32IN>(a.w, idx, baseV / Dv + (int64_t)(t0 + rr) * H, a.scalar_w, ww);
          if (a.raw_gates) {
#pragma unroll
            for (int q = 0; q < 8; ++q) ww[q] = sigmoid_f(ww[q]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) vv[q] = ww[q] = 0.f;
        }
        const int rs = rr ^ (8 * (j8 & Cfg::kWvSwz));  // rows 8 * j8 + q: (row / 8) = j8
#pragma unroll
        for (int q = 0; q < 8; ++q) sWVT[(8 * j8 + q) * LDC + rs] = static_cast<OpT>(ww[q] * vv[q]);
      }
    }
  }

  // pre-activation decay: log_alpha = -softplus(input) on the sequence's rows
  // (after every load is issued, so the loads stay in flight together)
  if (a.raw_gates && live && r < Lr) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[sl][j] = neg_softplus_f(g[sl][j]);
  }
  // per-token log-decay floor (padding rows hold 0)
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
    for (int j = 0; j < 4; ++j) g[sl][j] = la_floor(g[sl][j]);

  // ---- gates: inclusive cumsum over the rows of the chunk ----
  // within the wave (rows r = lane / TPR of this wave), then across waves
#pragma unroll
  for (int off = TPR; off < kWave; off *= 2) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = __shfl_up(g[sl][j], off, kWave);
        if (l >= off) g[sl][j] += y;
      }
  }
  if (l >= kWave - TPR) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
      *reinterpret_cast<float4*>(sTot + wid * DK + sl * SW + 4 * c4) = make_float4(g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
  }
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    float4 off = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int w2 = 0; w2 < wid; ++w2) {
      const float4 t4 = *reinterpret_cast<const float4*>(sTot + w2 * DK + sl * SW + 4 * c4);
      off.x += t4.x; off.y += t4.y; off.z += t4.z; off.w += t4.w;
    }
    g[sl][0] += off.x; g[sl][1] += off.y; g[sl][2] += off.z; g[sl][3] += off.w;
    const int c0 = sl * SW + 4 * c4;
    if (r == C / 2 - 1) *reinterpret_cast<float4*>(sCh + c0) = make_float4(g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
    if (r == C - 1) *reinterpret_cast<float4*>(sCh + DK + c0) = make_float4(g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
  }
  __syncthreads();
  // a wide-decay chunk: on some channel the cumulative decay from the chunk middle leaves the range
  // that the middle-referenced factors can carry (gdn2_wide.h)
  bool far = false;
  if (!WIDE && live) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int j = 0; j < 4; ++j) far = far || fabsf(g[sl][j] - sCh[sl * SW + 4 * c4 + j]) > kWideSpan;
  }
  for (int c = tid; c < DK; c += NT) {
    sCh[2 * DK + c] = __expf(sCh[c]);
    sCh[3 * DK + c] = __expf(sCh[DK + c] - sCh[c]);
  }
  float* sBs = reinterpret_cast<float*>(smem + Cfg::oBS);
  float* sPS = reinterpret_cast<float*>(smem + Cfg::oPS);
  if constexpr (!WIDE) {
    const bool wide = __builtin_amdgcn_readfirstlane(__syncthreads_or(far)) != 0;  // uniform: a scalar branch
    if (tid == 0) {
      *reinterpret_cast<int*>(rec + wide_flag_offset<Rec>()) = wide ? 1 : 0;
      if constexpr (DIR == 2) *reinterpret_cast<int*>(recB + wide_flag_offset<RecB>()) = wide ? 1 : 0;
    }
    if (wide) return;  // the whole workgroup: the wide pass writes this chunk's record
  } else {
    __syncthreads();
    // g <- cumulative log-decay from the start of the row's 16-token block, from the log-decays
    // again (no difference of two long sums is ever formed); block totals; pair scales
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int c0 = sl * SW + 4 * c4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live && r < Lr) {
        const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c0;
        x = load_la4(a.log_alpha, idx, baseK / DK + (int64_t)(t0 + r) * H, a.scalar_decay);
      }
      g[sl][0] = x.x; g[sl][1] = x.y; g[sl][2] = x.z; g[sl][3] = x.w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (a.raw_gates && live && r < Lr) g[sl][j] = neg_softplus_f(g[sl][j]);
        g[sl][j] = la_floor(g[sl][j]);
      }
    }
#pragma unroll
    for (int off = TPR; off < kWave; off *= 2) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = __shfl_up(g[sl][j], off, kWave);
          if (l >= off) g[sl][j] += y;
        }
    }
    if constexpr (Cfg::RPW < 16) {  // a 16-token block spans two waves: the odd one adds the even one's total
      if (l >= kWave - TPR) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
          *reinterpret_cast<float4*>(sTot + wid * DK + sl * SW + 4 * c4) =
              make_float4(g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
      }
      __syncthreads();
      if (wid & 1) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          const float4 t4 = *reinterpret_cast<const float4*>(sTot + (wid - 1) * DK + sl * SW + 4 * c4);
          g[sl][0] += t4.x; g[sl][1] += t4.y; g[sl][2] += t4.z; g[sl][3] += t4.w;
        }
      }
    }
    if (live && (r & 15) == 15) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
        *reinterpret_cast<float4*>(sBs + (r >> 4) * DK + sl * SW + 4 * c4) =
            make_float4(g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
    }
    __syncthreads();
    wide_pair_scales<NB, DK, NT>(sBs, sPS);
    __syncthreads();
  }

  // ---- factors and the Gram products, one channel slice at a time ----
  // A tiles (R, I) from Kh' Kt'^T; the causal term as P^T tiles (I, R) from
  // Kt' Qh'^T, whose accumulators are P's record units directly
  f32x4 accG[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) accG[i] = zero4();
  constexpr int LDW = Cfg::LDW;
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const int cl = 4 * c4, c0 = sl * SW + cl;
    float wbk[4] = {0.f, 0.f, 0.f, 0.f}, wq[4] = {0.f, 0.f, 0.f, 0.f};  // WIDE: b k and q of the row
    if (live) {
      float qv[4], kv[4], bv[4];
      cvt(rq[sl], qv);
      cvt(rk[sl], kv);
      cvt(rb[sl], bv);
      if (a.raw_gates) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = sigmoid_f(bv[i]);  // k is zero on padding rows
      }
      float khm[4], qhm[4], ktm[4], qs[4], kb[4], kh[4];
      if constexpr (!WIDE) {
        const float4 gm4 = *reinterpret_cast<const float4*>(sCh + c0);
        const float4 eg4 = *reinterpret_cast<const float4*>(sCh + 2 * DK + c0);
        const float4 ec4 = *reinterpret_cast<const float4*>(sCh + 3 * DK + c0);
        const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
        const float egm[4] = {eg4.x, eg4.y, eg4.z, eg4.w}, egcm[4] = {ec4.x, ec4.y, ec4.z, ec4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e1 = __expf(g[sl][i] - gm[i]);     // exp(g - g_m)
          const float e2 = __builtin_amdgcn_rcpf(e1);     // exp(g_m - g)
          khm[i] = bv[i] * kv[i] * e1;
          qhm[i] = qv[i] * e1;
          ktm[i] = kv[i] * e2;
          qs[i] = qv[i] * e1 * egm[i];                    // q exp(g)
          kb[i] = kv[i] * egcm[i] * e2;                   // k exp(g_C - g)
          kh[i] = khm[i] * egm[i];                        // b k exp(g)
        }
      } else {
        // block-referenced factors (all <= 1): rows at their block start, columns at their block end
        const int R = r >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gb = g[sl][i], bs = sBs[R * DK + c0 + i];
          const float E = __expf(gb), Fc = __expf(bs - gb);
          const float eg = __expf(wide_before<NB, DK>(sBs, R, c0 + i) + gb);        // exp(g)
          const float ec = __expf((bs - gb) + wide_after<NB, DK>(sBs, R, c0 + i));  // exp(g_C - g)
          wbk[i] = bv[i] * kv[i];
          wq[i] = qv[i];
          khm[i] = wbk[i] * E;
          qhm[i] = qv[i] * E;
          ktm[i] = kv[i] * Fc;
          qs[i] = qv[i] * eg;
          kb[i] = kv[i] * ec;
          kh[i] = wbk[i] * eg;
        }
      }
      // the token-major factor (forward: decayed q; backward: k decayed to the
      // chunk end) straight into its record units; the channel-major one
      // (forward: k decayed to the chunk end; backward: decayed q) staged transposed.
      // DIR 2 writes both token-major factors and stages the forward's channel-major
      // one here, the backward's after the inversion.
      {
        const float* tm = DIR == 1 ? kb : qs;
        const float* cm = DIR == 1 ? qs : kb;
#pragma unroll
        for (int i = 0; i < 4; ++i) sT1[(c0 + i) * LDC + r] = static_cast<OpT>(cm[i]);
        auto put = [&](char* rbase, int ubase, const float (&x)[4]) {
          char* dst = rbase + ubase * F::kUnitBytes + unit_off4<F32IN>(r, c0, Rec::UK);
          if constexpr (F32IN) {
            *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
          } else {
            f16x4 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(x[i]);
            *reinterpret_cast<f16x4*>(dst) = hv;
            if (DK < 32) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(0u, 0u);  // unit wider than Dk
          }
        };
        float tmv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tmv[i] = tm[i];
        put(rec, Rec::u1, tmv);
        if constexpr (DIR == 2) put(recB, RecB::u1, kb);
        if constexpr (DIR != 0) put(recB, RecB::u5, kh);  // b k exp(g) for the gradient kernel
      }
      if constexpr (WIDE) {
        float* s0 = reinterpret_cast<float*>(sSL) + r * LDW + cl;
        st4(s0 + 0 * (C * LDW), khm[0], khm[1], khm[2], khm[3]);
        st4(s0 + 1 * (C * LDW), qhm[0], qhm[1], qhm[2], qhm[3]);
        st4(s0 + 2 * (C * LDW), ktm[0], ktm[1], ktm[2], ktm[3]);
      } else if constexpr (F32IN) {
        float* s0 = reinterpret_cast<float*>(sSL) + r * LDSW + cl;
        st4(s0 + 0 * (C * LDSW), khm[0], khm[1], khm[2], khm[3]);
        st4(s0 + 1 * (C * LDSW), qhm[0], qhm[1], qhm[2], qhm[3]);
        st4(s0 + 2 * (C * LDSW), ktm[0], ktm[1], ktm[2], ktm[3]);
      } else {
        __bf16* s0 = reinterpret_cast<__bf16*>(sSL) + r * LDSW + cl;
        const float* src[3] = {khm, qhm, ktm};
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          float hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = bf16_to_f32(f32_to_bf16(src[p][i]));
            lo[i] = src[p][i] - hi[i];
          }
          st4(s0 + (2 * p) * (C * LDSW), hi[0], hi[1], hi[2], hi[3]);
          st4(s0 + (2 * p + 1) * (C * LDSW), lo[0], lo[1], lo[2], lo[3]);
        }
      }
    }
    __syncthreads();
    if constexpr (!WIDE) {
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int t = wid + NW * i;
        if (t < NGT2) {
          int R, I;
          const int kind = gram_tile<DIR, NGT>(t, R, I);
          const bool isP = kind != 0;
          if constexpr (F32IN) {
            const float* sl0 = reinterpret_cast<const float*>(sSL);
            const float* Kh = sl0;
            const float* Qh = sl0 + C * LDSW;
            const float* Kt = sl0 + 2 * (C * LDSW);
            if (kind == 1) mma_nt_k<SW>(accG[i], Kt + 16 * I * LDSW, LDSW, Qh + 16 * R * LDSW, LDSW);
            else if (isP) mma_nt_k<SW>(accG[i], Qh + 16 * R * LDSW, LDSW, Kt + 16 * I * LDSW, LDSW);
            else mma_nt_k<SW>(accG[i], Kh + 16 * R * LDSW, LDSW, Kt + 16 * I * LDSW, LDSW);
          } else {
            const __bf16* sl0 = reinterpret_cast<const __bf16*>(sSL);
            const __bf16* Kh = sl0;
            const __bf16* Qh = sl0 + 2 * (C * LDSW);
            const __bf16* Kt = sl0 + 4 * (C * LDSW);
            if (kind == 1)
              mma_nt_split_k<SW>(accG[i], Kt + 16 * I * LDSW, Kt + C * LDSW + 16 * I * LDSW, LDSW,
                                 Qh + 16 * R * LDSW, Qh + C * LDSW + 16 * R * LDSW, LDSW);
            else if (isP)
              mma_nt_split_k<SW>(accG[i], Qh + 16 * R * LDSW, Qh + C * LDSW + 16 * R * LDSW, LDSW,
                                 Kt + 16 * I * LDSW, Kt + C * LDSW + 16 * I * LDSW, LDSW);
            else
              mma_nt_split_k<SW>(accG[i], Kh + 16 * R * LDSW, Kh + C * LDSW + 16 * R * LDSW, LDSW,
                                 Kt + 16 * I * LDSW, Kt + C * LDSW + 16 * I * LDSW, LDSW);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    } else {
      // off-diagonal tiles on fp32 matrix cores from the block-referenced factors, the row
      // factor scaled by the decay of the blocks in between (pair scale)
      const float* Kh = reinterpret_cast<const float*>(sSL);
      const float* Qh = Kh + C * LDW;
      const float* Kt = Kh + 2 * (C * LDW);
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int t = wid + NW * i;
        if (t < NGT2) {
          int R, I;
          const int kind = gram_tile<DIR, NGT>(t, R, I);
          if (I < R) {
            const float* s = I + 2 <= R ? sPS + wide_pair(R, I) * DK + sl * SW : nullptr;
            if (kind == 1) mma_nt_f32s<SW>(accG[i], Kt + 16 * I * LDW, LDW, Qh + 16 * R * LDW, LDW, s);
            else if (kind == 2) mma_nt_f32s<SW>(accG[i], Qh + 16 * R * LDW, LDW, Kt + 16 * I * LDW, LDW, s);
            else mma_nt_f32s<SW>(accG[i], Kh + 16 * R * LDW, LDW, Kt + 16 * I * LDW, LDW, s);
          }
        }
      }
      __syncthreads();
      // diagonal blocks exactly, pair by pair: k and the block-relative decay of every row, then
      // the row sums into tables that the owners of the diagonal tiles add
      float* sKw = reinterpret_cast<float*>(sSL);
      float* sGw = sKw + C * LDW;
      float* tA = sGw + C * LDW;
      float* tP = tA + C * 16;
      if (live) {
        float kv[4];
        cvt(rk[sl], kv);
        st4(sKw + r * LDW + cl, kv[0], kv[1], kv[2], kv[3]);
        st4(sGw + r * LDW + cl, g[sl][0], g[sl][1], g[sl][2], g[sl][3]);
      }
      __syncthreads();
      {
        const float gbr[4] = {g[sl][0], g[sl][1], g[sl][2], g[sl][3]};
        gram_diag_pairwise<TPR, C>(r, live, cl, wbk, wq, gbr, sKw, sGw, LDW, tA, tP);
      }
      __syncthreads();
      {
        const int lr = l & 15, lg = l >> 4;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
          const int t = wid + NW * i;
          if (t < NGT2) {
            int R, I;
            const int kind = gram_tile<DIR, NGT>(t, R, I);
            if (I == R) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int ar = 16 * R + 4 * lg + e, ac = 16 * R + lr;  // accumulator row, column
                accG[i][e] += kind == 0 ? tA[ar * 16 + lr] : kind == 1 ? tP[ac * 16 + 4 * lg + e] : tP[ar * 16 + lr];
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- channel-major factor units; A -> LDS (strict lower); the causal term's
  //      units: forward P from P^T accumulators, backward P^T from P accumulators ----
  write_units<F32IN>(sT1, LDC, DK, C, rec + Rec::u2 * F::kUnitBytes, wid, NW);
  {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int t = wid + NW * i;
      if (t < NGT2) {
        int R, I;
        const int kind = gram_tile<DIR, NGT>(t, R, I);
        if (kind == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
            sAf[row * LDCF + col] = row > col ? accG[i][e] : 0.f;
          }
        } else {
          // forward accumulator: rows j = 16I + 4lg + e, column i = 16R + lr (keep j <= i),
          // unit row i; backward: rows i = 16R + 4lg + e, column j = 16I + lr (keep
          // j <= i), unit row j of P^T -- the same mask and offsets with (R, I) swapped
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool keep = kind == 1 ? (I < R || 4 * lg + e <= lr) : (I < R || lr <= 4 * lg + e);
            pv[e] = keep ? accG[i][e] : 0.f;
          }
          const int urow = kind == 1 ? 16 * R + lr : 16 * I + lr;
          const int ukk = kind == 1 ? 16 * I + 4 * lg : 16 * R + 4 * lg;
          char* dst = kind == 1 ? rec + Rec::u3 * F::kUnitBytes + unit_off4<F32IN>(urow, ukk, Rec::UC)
                                : recB + RecB::u0 * F::kUnitBytes + unit_off4<F32IN>(urow, ukk, RecB::UC);
          if constexpr (F32IN) {
            *reinterpret_cast<float4*>(dst) = make_float4(pv[0], pv[1], pv[2], pv[3]);
          } else {
            f16x4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(pv[e]);
            *reinterpret_cast<f16x4*>(dst) = hv;
            // the other half of a diagonal unit lies on the zero side of the diagonal
            // (forward: the next block; backward: the previous one) or past the chunk
            if (I == R) {
              if (kind == 1 && (R & 1) == 0) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(0u, 0u);
              if (kind == 2 && (R & 1) == 1) *reinterpret_cast<uint2*>(dst - 8) = make_uint2(0u, 0u);
              if (kind == 2 && (R & 1) == 0 && R + 1 == NB) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(0u, 0u);
            }
          }
        }
      }
    }
  }

  // ---- T = (I + A)^-1 ----
  KS ks;
  ks.invert(sAf, sXs);  // begins and ends with a barrier

  // ---- backward: T units for the per-chunk gradient kernel ----
  if constexpr (DIR != 0) write_units_f32<F32IN>(sAf, LDCF, C, C, recB + RecB::u4 * F::kUnitBytes, wid, NW);

  // ---- both records: the backward's channel-major factor (decayed q) through the
  //      same staging buffer, free since the inversion's first barrier ----
  if constexpr (DIR == 2) {
    if (live) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        const int c0 = sl * SW + 4 * c4;
        float qv[4];
        cvt(rq[sl], qv);
        const float4 gm4 = *reinterpret_cast<const float4*>(sCh + c0);
        const float4 eg4 = *reinterpret_cast<const float4*>(sCh + 2 * DK + c0);
        const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w}, egm[4] = {eg4.x, eg4.y, eg4.z, eg4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the same operations in the same order as the separate backward record pass (bitwise equal records)
          float qs;
          if constexpr (WIDE) {
            qs = qv[i] * __expf(wide_before<NB, DK>(sBs, r >> 4, c0 + i) + g[sl][i]);
          } else {
            const float e1 = __expf(g[sl][i] - gm[i]);
            qs = qv[i] * e1 * egm[i];
          }
          sT1[(c0 + i) * LDC + r] = static_cast<OpT>(qs);
        }
      }
    }
    __syncthreads();
    write_units<F32IN>(sT1, LDC, DK, C, recB + RecB::u2 * F::kUnitBytes, wid, NW);
    __syncthreads();
  }

  // ---- Kh^T = (b k exp(g))^T over the dead Kb^T staging ----
  if (live) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int c0 = sl * SW + 4 * c4;
      float kv[4], bv[4];
      cvt(rk[sl], kv);
      cvt(rb[sl], bv);
      if (a.raw_gates) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = sigmoid_f(bv[i]);  // k is zero on padding rows
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // g is block-relative on the wide path
        const float gg = WIDE ? wide_before<NB, DK>(sBs, r >> 4, c0 + i) + g[sl][i] : g[sl][i];
        sT1[(c0 + i) * LDC + r] = static_cast<OpT>(bv[i] * kv[i] * __expf(gg));
      }
    }
  }
  __syncthreads();

  // ---- forward: -W units from W^T tiles (channel blocks 2u, 2u+1, or u for fp32) ----
  if constexpr (DIR != 1) {
    constexpr int CPU = F32IN ? 1 : 2;
    constexpr int NWU = (C / 16) * Rec::UK;
    for (int t = wid; t < NWU; t += NW) {
      const int R = t / Rec::UK, u = t - R * Rec::UK;
      f32x4 w2[CPU];
#pragma unroll
      for (int p = 0; p < CPU; ++p) {
        w2[p] = zero4();
        const int cb = CPU * u + p;
        if (cb < DK / 16) mma_nt_yf32<OpT>(w2[p], sT1 + 16 * cb * LDC, LDC, sAf + 16 * R * LDCF, LDCF, 16 * (R + 1));
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
  }
  // ---- backward: -W^T units from W tiles (rows t, column d): the accumulator
  //      lane (d, g) holds tokens 4g+e, which are -W^T's unit slots ----
  if constexpr (DIR != 0) {
    const int lr = l & 15, lg = l >> 4;
    constexpr int NWT = (C / 16) * (DK / 16);
    for (int t = wid; t < NWT; t += NW) {
      const int R = t / (DK / 16), cb = t - R * (DK / 16);
      f32x4 acc = zero4();
      mma_nt_xf32<OpT>(acc, sAf + 16 * R * LDCF, LDCF, sT1 + 16 * cb * LDC, LDC, 16 * (R + 1));
      char* dst = recB + RecB::u3 * F::kUnitBytes + unit_off4<F32IN>(16 * cb + lr, 16 * R + 4 * lg, RecB::UC);
      if constexpr (F32IN) {
        *reinterpret_cast<float4*>(dst) = make_float4(-acc[0], -acc[1], -acc[2], -acc[3]);
      } else {
        f16x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(-acc[e]);
        *reinterpret_cast<f16x4*>(dst) = hv;
        if (C < 32) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(0u, 0u);  // unit wider than the chunk
      }
    }
  }
  for (int c = tid; c < DK; c += NT) {
    const float gc = __expf(sCh[DK + c]);
    reinterpret_cast<float*>(rec + Rec::uG * F::kUnitBytes)[c] = gc;
    if constexpr (DIR == 2) reinterpret_cast<float*>(recB + RecB::uG * F::kUnitBytes)[c] = gc;
  }

  // ---- Ut = T (w v): accumulator tiles straight to the workspace ----
  if constexpr (DIR != 1) {
    const int nvt = Dv / 16, ntile = (C / 16) * nvt;
    for (int t = wid; t < ntile; t += NW) {
      const int R = t / nvt, jb = t - R * nvt;
      f32x4 acc = zero4();
      mma_nt_xf32<OpT>(acc, sAf + 16 * R * LDCF, LDCF, sWVT + 16 * jb * LDC, LDC, 16 * (R + 1), 16 * jb,
                       Cfg::kWvSwz);
      if constexpr (F32IN) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(ut) + (int64_t)t * 256 + 4 * l) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 h = {static_cast<_Float16>(acc[0]), static_cast<_Float16>(acc[1]), static_cast<_Float16>(acc[2]),
                      static_cast<_Float16>(acc[3])};
        *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(ut) + (int64_t)t * 256 + 4 * l) = h;
      }
    }
  }
}

// The record pass: one workgroup per chunk on the fast path (two per CU at d_k = 128, chunk 64).
// The LDS of the wide-path tables is not part of it.
template <int DK, int C, bool F32IN, int DIR>
__global__ __launch_bounds__(512, 4) void gdn2_prep_kernel(FwdArgs a, char* rec_base, float* ut_base,
                                                            char* brec_base) {
  __shared__ __attribute__((aligned(16))) char smem[PrepCfg<DK, C, F32IN, DIR>::oBS];
  prep_chunk<DK, C, F32IN, DIR, false>(a, rec_base, ut_base, brec_base,
                                       chunk_item_of_block(a.vl, a.T, a.H, C, blockIdx.x), smem);
}

// The chunks the record pass flagged as wide-decay, recomputed exactly. Workgroup w covers items
// w, w + gridDim.x, ...: it reads their flags in parallel, lists the flagged ones in LDS and
// processes them one after another (each result depends on its chunk alone, so the list order
// does not matter). With no wide chunk every workgroup only reads its flags.
template <int DK, int C, bool F32IN, int DIR>
__global__ __launch_bounds__(512) void gdn2_prep_wide_kernel(FwdArgs a, char* rec_base, float* ut_base,
                                                              char* brec_base, int nitems) {
  using Cfg = PrepCfg<DK, C, F32IN, DIR>;
  using Rec = typename Cfg::Rec;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  __shared__ int list[kWideBatch];
  __shared__ int count;
  const int per = (nitems + (int)gridDim.x - 1) / (int)gridDim.x;
  for (int k0 = 0; k0 < per; k0 += kWideBatch) {
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    const int k = k0 + (int)threadIdx.x;
    const int64_t item = blockIdx.x + (int64_t)k * gridDim.x;
    if (threadIdx.x < kWideBatch && k < per && item < nitems) {
      const int f = *reinterpret_cast<const int*>(rec_base + item * Rec::kBytes + wide_flag_offset<Rec>());
      if (f == 1) list[atomicAdd(&count, 1)] = (int)item;
    }
    __syncthreads();
    const int n = count;
    for (int j = 0; j < n; ++j) {
      prep_chunk<DK, C, F32IN, DIR, true>(a, rec_base, ut_base, brec_base, list[j], smem);
      __syncthreads();
    }
    __syncthreads();
  }
}

template <int DK, int C, bool F32IN, int DIR>
static hipError_t launch_prep_t(const FwdArgs& a, char* rec, float* ut, char* brec, hipStream_t s) {
  if constexpr (!PrepCfg<DK, C, F32IN, DIR>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int64_t grid = chunk_items(a.vl, a.B, a.T, a.H, C);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gdn2_prep_kernel<DK, C, F32IN, DIR>), dim3((unsigned)grid), dim3(512), 0, s, a, rec, ut,
                       brec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int wgrid = grid < kWideGrid ? (int)grid : kWideGrid;
    hipLaunchKernelGGL((gdn2_prep_wide_kernel<DK, C, F32IN, DIR>), dim3((unsigned)wgrid), dim3(512), 0, s, a, rec,
                       ut, brec, (int)grid);
    return hipGetLastError();
  }
}

template <int DK, bool F32IN, int DIR>
static hipError_t launch_prep_c(const FwdArgs& a, char* rec, float* ut, char* brec, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_prep_t<DK, 16, F32IN, DIR>(a, rec, ut, brec, s);
    case 32: return launch_prep_t<DK, 32, F32IN, DIR>(a, rec, ut, brec, s);
    case 64: return launch_prep_t<DK, 64, F32IN, DIR>(a, rec, ut, brec, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN, int DIR>
static hipError_t launch_prep_f(const FwdArgs& a, char* rec, float* ut, char* brec, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_prep_c<16, F32IN, DIR>(a, rec, ut, brec, s);
    case 32: return launch_prep_c<32, F32IN, DIR>(a, rec, ut, brec, s);
    case 64: return launch_prep_c<64, F32IN, DIR>(a, rec, ut, brec, s);
    case 128: return launch_prep_c<128, F32IN, DIR>(a, rec, ut, brec, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prep_fwd(const FwdArgs& a, char* rec, float* ut, hipStream_t s) {
  return a.f32_inputs ? launch_prep_f<true, 0>(a, rec, ut, nullptr, s)
                      : launch_prep_f<false, 0>(a, rec, ut, nullptr, s);
}

hipError_t launch_prep_bwd(const FwdArgs& a, char* rec, hipStream_t s) {
  return a.f32_inputs ? launch_prep_f<true, 1>(a, rec, nullptr, nullptr, s)
                      : launch_prep_f<false, 1>(a, rec, nullptr, nullptr, s);
}

hipError_t launch_prep_train(const FwdArgs& a, char* rec, float* ut, char* brec, hipStream_t s) {
  return a.f32_inputs ? launch_prep_f<true, 2>(a, rec, ut, brec, s) : launch_prep_f<false, 2>(a, rec, ut, brec, s);
}

template <int DK, bool F32IN>
static bool prep_fits_c(int chunk) {
  switch (chunk) {
    case 16: return PrepCfg<DK, 16, F32IN, 0>::kFits && PrepCfg<DK, 16, F32IN, 1>::kFits &&
                    PrepCfg<DK, 16, F32IN, 2>::kFits;
    case 32: return PrepCfg<DK, 32, F32IN, 0>::kFits && PrepCfg<DK, 32, F32IN, 1>::kFits &&
                    PrepCfg<DK, 32, F32IN, 2>::kFits;
    case 64: return PrepCfg<DK, 64, F32IN, 0>::kFits && PrepCfg<DK, 64, F32IN, 1>::kFits &&
                    PrepCfg<DK, 64, F32IN, 2>::kFits;
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

size_t record_bytes(int Dk, int chunk, bool f32, int dir) {
#define GDN2_REC(DK, CC)                                                                            \
  if (Dk == DK && chunk == CC) {                                                                    \
    if (dir == 0) return f32 ? (size_t)Record<DK, CC, true, 0>::kBytes : (size_t)Record<DK, CC, false, 0>::kBytes; \
    return f32 ? (size_t)Record<DK, CC, true, 1>::kBytes : (size_t)Record<DK, CC, false, 1>::kBytes;  \
  }
  GDN2_REC(16, 16) GDN2_REC(16, 32) GDN2_REC(16, 64)
  GDN2_REC(32, 16) GDN2_REC(32, 32) GDN2_REC(32, 64)
  GDN2_REC(64, 16) GDN2_REC(64, 32) GDN2_REC(64, 64)
  GDN2_REC(128, 16) GDN2_REC(128, 32) GDN2_REC(128, 64)
#undef GDN2_REC
  return 0;
}

size_t fwd_record_bytes(int Dk, int chunk, bool f32) { return record_bytes(Dk, chunk, f32, 0); }

}  // namespace gdn2
