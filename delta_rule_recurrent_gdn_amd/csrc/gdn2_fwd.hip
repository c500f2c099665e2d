// gdn2_fwd.hip -- chunkwise WY forward of the Gated Delta Rule-2 operator.
//
// Method: the chunkwise WY algorithm with the channel-wise decay absorbed into
// asymmetric erase factors (arXiv 2605.22791 abstract; research-wiki summary,
// "Key findings"). For a chunk of C tokens entered with state S (Dk x Dv),
// local token index r, cumulative in-chunk log-decay g_r = sum_{i<=r} log_alpha_i:
//
//   Kh = exp(g) * b * k          left erase factor (decayed erase key)
//   Kt = k * exp(-g)             right erase factor (inverse-decayed key)
//   A  = strict_lower(Kh Kt^T),  T = (I + A)^-1          (unit lower triangular)
//   W  = T Kh,   U = T (w * v) - W S                     (WY factors; U are the
//                                                         per-token writes u_r)
//   P  = lower_incl((q * exp(g)) Kt^T)
//   O  = (q * exp(g)) S + P U
//   S <- Diag(exp(g_C)) S + (k * exp(g_C - g))^T U
//
// This is an exact refactoring of the token-by-token recurrence
// S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T, o_t = S_t^T q_t
// (the GatedDeltaNet-2 README update-rule paragraph; arXiv abstract): unrolling the
// recurrence inside the chunk gives (I + A) U = w*v - Kh S.
//
// One workgroup owns one (batch, head, value tile of BV columns) and walks the
// chunks in order with its fp32 state tile resident in matrix-core accumulators.
// Value columns of the state evolve independently (every operator acts on S
// from the left), so value tiles need no communication. The two value tiles of
// one head are placed on the same XCD so their shared key-side reads hit that
// XCD's L2.
//
// Per chunk the workgroup performs
//   (1) gate preprocessing: log_alpha rows -> LDS, in-chunk inclusive cumsum per
//       channel (g), plus g at the last and the middle token;
//   (2) factors: decay-scaled q, k, b*k into LDS operand buffers; the Gram
//       factors for A and P are referenced to the chunk middle so that the
//       exp(+-g) pairs stay in range;
//   (3) A and P on matrix cores, T = (I + A)^-1 by blocked forward substitution
//       (16x16 diagonal blocks by substitution in registers, off-diagonal blocks
//       by two levels of block products);
//   (4) W and T (w*v) on matrix cores, then the sequential part: U, O and the
//       state update.
//
// Precision (bf16 inputs): the Gram matrices A and P are formed from a two-term
// bf16 split of their decay-scaled operands (wide exponent range, ~16-bit
// mantissa); every other operand is fp16 (the values are bounded by 1 or by the
// magnitude of v and S); accumulation, the state and g are fp32. fp32 inputs
// use fp32 matrix-core products throughout.

#include "gdn2_chunk.h"
#include "gdn2_internal.h"

namespace gdn2 {

// Workgroup size: 8 waves (two per SIMD) hide each other's LDS and matrix-core
// latencies; every wave has 256 registers.
constexpr int kFwdThreads = 512;

template <int DK, int C, int BV, bool F32IN>
struct FwdCfg {
  static constexpr int kThreads = kFwdThreads;
  using KS = KSide<DK, C, F32IN, kThreads>;
  using OpT = typename KS::OpT;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int NB = KS::NB;
  static constexpr int LDC = KS::LDC, LDK = KS::LDK, LDCF = KS::LDCF, LDX = KS::LDX;
  static constexpr int OPB = sizeof(OpT);

  // persistent region
  static constexpr int oKhT = 0;                                   // OpT [DK][LDC]  (b k exp(g))^T
  static constexpr int oQs = oKhT + DK * LDC * OPB;                // OpT [C][LDK]   q exp(g)
  static constexpr int oKbT = oQs + C * LDK * OPB;                 // OpT [DK][LDC]  (k exp(g_C - g))^T
  static constexpr int oWVT = oKbT + DK * LDC * OPB;               // OpT [BV][LDC]  (w v)^T
  static constexpr int oST = oWVT + BV * LDC * OPB;                // OpT [BV][LDK]  S^T
  static constexpr int oCH = oST + BV * LDK * OPB;                 // float [4][DK]  per-channel gate constants
  static constexpr int oTOT = oCH + KS::kChanBytes;                // float cumsum segment totals
  static constexpr int oBS = oTOT + KS::kTotBytes;                 // float [NB][DK] block totals (wide chunks)
  static constexpr int oPS = oBS + NB * DK * 4;                    // float [npair][DK] pair scales (wide chunks)
  static constexpr int oX = oPS + wide_npair(NB) * DK * 4;         // start of the phase-shared region
  // phase F (gate preprocessing + Gram)
  static constexpr int oG = oX;
  static constexpr int oSL = oG + KS::kGBytes;
  // wide-decay chunks use the slice region for b k, q and k of one channel slice (fp32 [C][LDW]
  // each), then for the diagonal-block tables of A and P ([C][16] each)
  static constexpr int LDW = KS::SW + 4;
  static constexpr int kWideSl = 3 * C * LDW * 4 > 2 * C * 16 * 4 ? 3 * C * LDW * 4 : 2 * C * 16 * 4;
  static constexpr int endF = oSL + (KS::kSlicesBytes > kWideSl ? KS::kSlicesBytes : kWideSl);
  // phase W (after the Gram products)
  static constexpr int oAf = oX;                                   // float [C][LDCF]  A, then T
  static constexpr int oPm = oAf + KS::kAfBytes;                   // OpT [C][LDC]   P
  static constexpr int oWm = oPm + C * LDC * OPB;                  // OpT [C][LDK]   -W
  static constexpr int oUT = oWm + C * LDK * OPB;                  // OpT [BV][LDC]  U^T
  static constexpr int oXs = oUT + BV * LDC * OPB;                 // float inversion scratch
  static constexpr int endW = oXs + KS::kXsBytes;
  static constexpr int kLdsBytes = endF > endW ? endF : endW;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;

  static constexpr int NUT = NB * (BV / 16);                       // U / O tiles
  static constexpr int UPW = (NUT + kWaves - 1) / kWaves;
  static constexpr int NST = (DK / 16) * (BV / 16);                // state tiles
  static constexpr int SPW = (NST + kWaves - 1) / kWaves;
  static constexpr int NWT = (DK / 16) * NB;                       // W^T tiles
  static constexpr int WPW = (NWT + kWaves - 1) / kWaves;
  // v, w: 8 consecutive value columns of one row; rows vw_r + i * VW_RPP
  static constexpr int VW_RPP = kThreads / (BV / 8);
  static constexpr int VW_RPT = (C + VW_RPP - 1) / VW_RPP;
};

// A wide-decay chunk (gdn2_wide.h): its Gram matrices and decayed key-side
// operands with block-referenced decay factors, in place of KSide::factors_gram
// and gram_store -- A -> sAf (strict lower), P -> sPm (row-major, lower incl.),
// q exp(g) -> sQs, (b k exp(g))^T -> sKhT, (k exp(g_C - g))^T -> sKbT. The
// chunk's inputs are read again from global memory and every intermediate
// lives in LDS.
template <int DK, int C, int BV, bool F32IN, bool FL>
__device__ __forceinline__ void fwd_wide_chunk(const FwdArgs& a, int64_t baseK, int t0, int Lr, char* smem) {
  using Cfg = FwdCfg<DK, C, BV, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  constexpr int NT = kFwdThreads, NW = Cfg::kWaves, NB = Cfg::NB;
  constexpr int SW = KS::SW, NSL = KS::NSL, NGT = KS::NGT, GPW = KS::GPW;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDW = Cfg::LDW;
  OpT* sKhT = reinterpret_cast<OpT*>(smem + Cfg::oKhT);
  OpT* sQs = reinterpret_cast<OpT*>(smem + Cfg::oQs);
  OpT* sKbT = reinterpret_cast<OpT*>(smem + Cfg::oKbT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  float* sW = reinterpret_cast<float*>(smem + Cfg::oSL);
  float* sBs = reinterpret_cast<float*>(smem + Cfg::oBS);
  float* sPS = reinterpret_cast<float*>(smem + Cfg::oPS);
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  OpT* sPm = reinterpret_cast<OpT*>(smem + Cfg::oPm);
  // the wave index in a scalar register: per-wave branches and offsets stay scalar (B8 H16 T4096 single-pass
  // forward 1.34 -> 1.24 ms, training forward 0.86 -> 0.84 ms)
  const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int H = a.H;
  const int64_t rowK = (int64_t)H * DK, baseS = baseK / DK;
  const bool raw = FL && a.raw_gates, sla = FL && a.scalar_decay, sbg = FL && a.scalar_b;

  // log-decay (floored), then the cumulative sum inside each 16-token block and the block totals
#pragma unroll 1
  for (int e = tid; e < C * DK; e += NT) {
    const int r = e / DK, c = e - r * DK;
    float x = 0.f;
    if (r < Lr) {
      x = a.log_alpha[sla ? baseS + (int64_t)(t0 + r) * H : baseK + (int64_t)(t0 + r) * rowK + c];
      if (raw) x = neg_softplus_f(x);
      x = la_floor(x);
    }
    sG[e] = x;
  }
  __syncthreads();
#pragma unroll 1
  for (int e = tid; e < NB * DK; e += NT) {
    const int R = e / DK, c = e - R * DK;
    float run = 0.f;
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
      run += sG[(16 * R + i) * DK + c];
      sG[(16 * R + i) * DK + c] = run;
    }
    sBs[e] = run;
  }
  __syncthreads();
  wide_pair_scales<NB, DK, NT>(sBs, sPS);
  __syncthreads();

  // per channel slice: b k, q and k (fp32) and the decayed key-side operands; the off-diagonal
  // Gram tiles on fp32 matrix cores with the block-referenced decay factors applied as the
  // operands are read; the diagonal blocks pair by pair, thread (row r, columns j and j + 8)
  float* sBK = sW;
  float* sQ = sW + C * LDW;
  float* sK = sW + 2 * C * LDW;
  f32x4 accG[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) accG[i] = zero4();
  const int pr = tid / 8, pj = tid % 8;  // pairwise: row pr (< C), block columns pj and pj + 8
  float da0 = 0.f, da1 = 0.f, dp0 = 0.f, dp1 = 0.f;
#pragma unroll 1
  for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll 1
    for (int e = tid; e < C * SW; e += NT) {
      const int r = e / SW, cs = e - r * SW, c = sl * SW + cs;
      float qv = 0.f, kv = 0.f, bv = 0.f;
      if (r < Lr) {
        const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c;
        qv = load1<F32IN>(a.q, idx);
        kv = load1<F32IN>(a.k, idx);
        bv = load1<F32IN>(a.b, sbg ? baseS + (int64_t)(t0 + r) * H : idx);
        if (raw) bv = sigmoid_f(bv);
      }
      const int R = r >> 4;
      const float gb = sG[r * DK + c], bs = sBs[R * DK + c];
      const float eg = __expf(wide_before<NB, DK>(sBs, R, c) + gb);        // exp(g)
      const float ec = __expf((bs - gb) + wide_after<NB, DK>(sBs, R, c));  // exp(g_C - g)
      sBK[r * LDW + cs] = bv * kv;
      sQ[r * LDW + cs] = qv;
      sK[r * LDW + cs] = kv;
      sQs[r * LDK + c] = static_cast<OpT>(qv * eg);
      sKhT[c * LDC + r] = static_cast<OpT>(bv * kv * eg);
      sKbT[c * LDC + r] = static_cast<OpT>(kv * ec);
    }
    __syncthreads();
    // off-diagonal tiles: acc += sum_c (X_rc exp(gb_rc)) s_RI,c (k_ic exp(Bs_I,c - gb_ic))
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int t = wid + NW * i;
      if (t < NGT) {
        const bool isP = t >= NGT / 2;
        int R, I;
        tri_index(isP ? t - NGT / 2 : t, R, I);
        if (I < R) {
          const float* X = isP ? sQ : sBK;
          const int rr = 16 * R + lr, ii = 16 * I + lr;
#pragma unroll 1
          for (int k0 = 0; k0 < SW; k0 += 4) {
            const int c = sl * SW + k0 + lg;
            float x = X[rr * LDW + k0 + lg] * __expf(sG[rr * DK + c]);
            if (I + 2 <= R) x *= sPS[wide_pair(R, I) * DK + c];
            const float y = sK[ii * LDW + k0 + lg] * __expf(sBs[I * DK + c] - sG[ii * DK + c]);
            accG[i] = mfma16x16x4(x, y, accG[i]);
          }
        }
      }
    }
    // diagonal blocks: A_ri and P_ri for i = 16 (r / 16) + pj and + 8, over the slice's channels
    if (pr < C) {
      const int rb = pr & ~15, rl = pr & 15;
#pragma unroll 1
      for (int cs = 0; cs < SW; ++cs) {
        const int c = sl * SW + cs;
        const float gr = sG[pr * DK + c], bkr = sBK[pr * LDW + cs], qr = sQ[pr * LDW + cs];
        if (pj <= rl) {
          const int i = rb + pj;
          const float t = sK[i * LDW + cs] * __expf(gr - sG[i * DK + c]);
          da0 += pj < rl ? bkr * t : 0.f;
          dp0 += qr * t;
        }
        if (pj + 8 <= rl) {
          const int i = rb + pj + 8;
          const float t = sK[i * LDW + cs] * __expf(gr - sG[i * DK + c]);
          da1 += pj + 8 < rl ? bkr * t : 0.f;
          dp1 += qr * t;
        }
      }
    }
    __syncthreads();
  }
  // the diagonal blocks into the owners' accumulators
  float* tA = sW;
  float* tP = sW + C * 16;
  if (pr < C) {
    tA[pr * 16 + pj] = da0;
    tA[pr * 16 + pj + 8] = da1;
    tP[pr * 16 + pj] = dp0;
    tP[pr * 16 + pj + 8] = dp1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int t = wid + NW * i;
    if (t < NGT) {
      const bool isP = t >= NGT / 2;
      int R, I;
      tri_index(isP ? t - NGT / 2 : t, R, I);
      if (I == R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) accG[i][e] += (isP ? tP : tA)[(16 * R + 4 * lg + e) * 16 + lr];
      }
    }
  }
  __syncthreads();
  KS().template gram_store<false>(accG, sAf, sPm);
}

// FL: some gate option (pre-activation or per-head scalar gates) is on; without
// it every gate-option branch of the loads folds away.
//
// The chunk loop of one workgroup, from S0. EXACT = false: no code for
// wide-decay chunks; a sequence that has one is computed to the end regardless
// (its results from that chunk on are wrong) and marked by kWideMark in the
// first value column of its last output row. EXACT = true (the second kernel):
// only marked sequences, every chunk, the wide ones through fwd_wide_chunk; it
// rewrites all of the sequence's outputs, the marked word included. Two kernels
// rather than one with a second loop exit or a call: either costs the fast
// loop's register allocation more spills than the rare sequence costs.
template <int DK, int C, int BV, bool F32IN, bool FL, bool EXACT>
__device__ __forceinline__ void fwd_chunks(const FwdArgs& a, char* smem) {
  using Cfg = FwdCfg<DK, C, BV, F32IN>;
  using KS = typename Cfg::KS;
  using OpT = typename Cfg::OpT;
  constexpr int NW = Cfg::kWaves, NB = Cfg::NB;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDCF = Cfg::LDCF;
  OpT* sKhT = reinterpret_cast<OpT*>(smem + Cfg::oKhT);
  OpT* sQs = reinterpret_cast<OpT*>(smem + Cfg::oQs);
  OpT* sKbT = reinterpret_cast<OpT*>(smem + Cfg::oKbT);
  OpT* sWVT = reinterpret_cast<OpT*>(smem + Cfg::oWVT);
  OpT* sST = reinterpret_cast<OpT*>(smem + Cfg::oST);
  float* sCh = reinterpret_cast<float*>(smem + Cfg::oCH);
  float* sTot = reinterpret_cast<float*>(smem + Cfg::oTOT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  OpT* sPm = reinterpret_cast<OpT*>(smem + Cfg::oPm);
  OpT* sWm = reinterpret_cast<OpT*>(smem + Cfg::oWm);
  OpT* sUT = reinterpret_cast<OpT*>(smem + Cfg::oUT);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);

  // the wave index in a scalar register: per-wave branches and offsets stay scalar (B8 H16 T4096 single-pass
  // forward 1.34 -> 1.24 ms, training forward 0.86 -> 0.84 ms)
  const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;

  // block -> (batch*head, value tile); the value tiles of one head share an XCD
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
  // the mark: the first value column of this workgroup's tile in the sequence's last output row
  const int64_t mark = baseV + (int64_t)(T - 1) * rowV;
  if constexpr (EXACT) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(__float_as_uint(a.o[mark]));
    if (m != kWideMark) return;
  }

  KS ks;
  ks.init(tid);
  const bool raw_gates = FL && a.raw_gates, scalar_w = FL && a.scalar_w;
  ks.raw = raw_gates;
  ks.scalar_la = FL && a.scalar_decay;
  ks.scalar_b = FL && a.scalar_b;
  constexpr int VW_RPP = Cfg::VW_RPP, VW_RPT = Cfg::VW_RPT;
  const int vw_r = tid / (BV / 8), vw_j8 = tid % (BV / 8);
  Raw8<F32IN> rv[VW_RPT], rw[VW_RPT];
  auto load_chunk = [&](int nn) {
    const int tn = nn * C, Ln = min(C, T - tn);
    ks.load(a.q, a.k, a.b, a.log_alpha, baseK, rowK, tn, Ln);
#pragma unroll
    for (int i = 0; i < VW_RPT; ++i) {
      const int r = vw_r + i * VW_RPP;
      if (r < Ln) {
        const int64_t idx = baseV + (int64_t)(tn + r) * rowV + 8 * vw_j8;
        ld_raw(rv[i], a.v, idx);
        ld_raw_gate(rw[i], a.w, idx, baseK / DK + (int64_t)(tn + r) * H, scalar_w);
      } else {
        zero_raw(rv[i]);
        zero_raw(rw[i]);
      }
    }
  };

  // ---- initial state: accumulators (fp32) and the operand copy S^T ----
  f32x4 accS[Cfg::SPW];
#pragma unroll
  for (int i = 0; i < Cfg::SPW; ++i) {
    const int t = wid + NW * i;
    accS[i] = zero4();
    if (t < Cfg::NST) {
      const int cb = t / (BV / 16), jb = t % (BV / 16);
      if (a.S0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accS[i][e] = a.S0[stBase + (int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr];
      }
      store_tile_t(sST + 16 * jb * LDK + 16 * cb, LDK, accS[i]);
    }
  }
  load_chunk(0);

  bool any_wide = false;
  for (int n = 0; n < NC; ++n) {
    const int t0 = n * C;
    const int Lr = min(C, T - t0);

    // entry states every state_every chunks (the caller's chunk when the kernel runs a finer one)
    if (a.chunk_states && n % a.state_every == 0) {
      const int ncs = (NC + a.state_every - 1) / a.state_every;
      float* cs = a.chunk_states + ((int64_t)bh * ncs + n / a.state_every) * DK * Dv + j0;
#pragma unroll
      for (int i = 0; i < Cfg::SPW; ++i) {
        const int t = wid + NW * i;
        if (t < Cfg::NST) {
          const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[(int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr] = accS[i][e];
        }
      }
    }
    __syncthreads();  // the previous chunk's readers of the per-chunk buffers are done

    // ---- (1) gate preprocessing; w*v -> sWVT ----
#pragma unroll
    for (int i = 0; i < VW_RPT; ++i) {
      const int r = vw_r + i * VW_RPP;
      if (r < C) {
        float vv[8], ww[8];
        cvt(rv[i], vv);
        cvt(rw[i], ww);
        if (raw_gates) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ww[e] = sigmoid_f(ww[e]);  // v is zero on padding rows
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sWVT[(8 * vw_j8 + e) * LDC + r] = static_cast<OpT>(ww[e] * vv[e]);
      }
    }
    // gates() also reports a wide-decay chunk: on some channel the cumulative decay from the chunk
    // middle leaves the range that the middle-referenced factors can carry (gdn2_wide.h)
    const bool wide = ks.gates(sTot, sG, sCh);
    if constexpr (!EXACT) any_wide = any_wide || wide;
    if (EXACT && wide) {
      fwd_wide_chunk<DK, C, BV, F32IN, FL>(a, baseK, t0, Lr, smem);
    } else {
      // ---- (2)+(3a) factors and the Gram products A, P ----
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
    }

    // ---- (3b) T = (I + A)^-1 ----
    ks.invert(sAf, sXs);

    // ---- (4a) W^T = Kh^T T^T -> sWm holds -W ; U tiles start as T (w*v) ----
#pragma unroll 1
    for (int i = 0; i < Cfg::WPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NWT) {
        const int cb = t / NB, R = t % NB;
        f32x4 acc = zero4();
        mma_nt_yf32<OpT>(acc, sKhT + 16 * cb * LDC, LDC, sAf + 16 * R * LDCF, LDCF, 16 * (R + 1));
        store_tile_t(sWm + 16 * R * LDK + 16 * cb, LDK, acc, -1.f);
      }
    }
    f32x4 accU[Cfg::UPW], accO[Cfg::UPW];
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      accU[i] = zero4();
      accO[i] = zero4();
      if (t < Cfg::NUT) {
        const int R = t / (BV / 16), jb = t % (BV / 16);
        mma_nt_xf32<OpT>(accU[i], sAf + 16 * R * LDCF, LDCF, sWVT + 16 * jb * LDC, LDC, 16 * (R + 1));
        // 16-bit inputs: T (w v) rounded to fp16, as the two-stage path stores it, so that both paths
        // round the same operands (U itself becomes an fp16 operand in every use)
        if constexpr (!F32IN) {
#pragma unroll
          for (int e = 0; e < 4; ++e) accU[i][e] = static_cast<float>(static_cast<_Float16>(accU[i][e]));
        }
      }
    }
    __syncthreads();

    // every raw input of this chunk is consumed: fetch the next chunk now so the
    // HBM latency overlaps the rest of this chunk's work
    if (n + 1 < NC) load_chunk(n + 1);

    // ---- (4b) U = T(w*v) - W S ; O = (q*exp(g)) S ----
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NUT) {
        const int R = t / (BV / 16), jb = t % (BV / 16);
        mma_nt_k<DK>(accU[i], sWm + 16 * R * LDK, LDK, sST + 16 * jb * LDK, LDK);
        if (a.o) mma_nt_k<DK>(accO[i], sQs + 16 * R * LDK, LDK, sST + 16 * jb * LDK, LDK);
        store_tile_t(sUT + 16 * jb * LDC + 16 * R, LDC, accU[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // ---- (4c) O += P U -> o ;  S <- Diag(exp(g_C)) S + Kb^T U ----
    if (a.o) {
#pragma unroll
      for (int i = 0; i < Cfg::UPW; ++i) {
        const int t = wid + NW * i;
        if (t < Cfg::NUT) {
          const int R = t / (BV / 16), jb = t % (BV / 16);
          mma_nt<OpT>(accO[i], sPm + 16 * R * LDC, LDC, sUT + 16 * jb * LDC, LDC, 16 * (R + 1));
          float* op = a.o + baseV + 16 * jb + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * R + 4 * lg + e;
            if (r < Lr) op[(int64_t)(t0 + r) * rowV] = accO[i][e];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NST) {
        const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= __expf(sCh[DK + 16 * cb + 4 * lg + e]);
        mma_nt_k<C>(accS[i], sKbT + 16 * cb * LDC, LDC, sUT + 16 * jb * LDC, LDC);
        store_tile_t(sST + 16 * jb * LDK + 16 * cb, LDK, accS[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (a.S_final) {
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NST) {
        const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.S_final[stBase + (int64_t)(16 * cb + 4 * lg + e) * Dv + 16 * jb + lr] = accS[i][e];
      }
    }
  }
  if constexpr (!EXACT) {
    if (any_wide) {  // after every wave's stores of the last row
      __syncthreads();
      if (tid == 0) a.o[mark] = __uint_as_float(kWideMark);
    }
  }
}

template <int DK, int C, int BV, bool F32IN, bool FL>
__global__ __launch_bounds__(kFwdThreads) void gdn2_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[FwdCfg<DK, C, BV, F32IN>::kLdsBytes];
  fwd_chunks<DK, C, BV, F32IN, FL, false>(a, smem);
}

// The sequences that the kernel above marked, recomputed exactly.
template <int DK, int C, int BV, bool F32IN, bool FL>
__global__ __launch_bounds__(kFwdThreads) void gdn2_fwd_exact_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[FwdCfg<DK, C, BV, F32IN>::kLdsBytes];
  fwd_chunks<DK, C, BV, F32IN, FL, true>(a, smem);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int DK, int C, int BV, bool F32IN>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  if constexpr (!FwdCfg<DK, C, BV, F32IN>::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int nv = a.Dv / BV;
    const int nbh = a.B * a.H;
    const int grid = ((nbh + 7) / 8) * 8 * nv;
    if (a.raw_gates || a.scalar_b || a.scalar_w || a.scalar_decay) {
      hipLaunchKernelGGL((gdn2_fwd_kernel<DK, C, BV, F32IN, true>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gdn2_fwd_exact_kernel<DK, C, BV, F32IN, true>), dim3(grid), dim3(kFwdThreads), 0, stream,
                         a);
    } else {
      hipLaunchKernelGGL((gdn2_fwd_kernel<DK, C, BV, F32IN, false>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gdn2_fwd_exact_kernel<DK, C, BV, F32IN, false>), dim3(grid), dim3(kFwdThreads), 0, stream,
                         a);
    }
    return hipGetLastError();
  }
}

// Value-tile width: the widest tile that still gives at least one workgroup per
// compute unit (256 CUs), never wider than Dv (and 32 at most for fp32 inputs,
// whose operands take twice the LDS).
static int pick_bv(int B, int H, int Dv, bool f32) {
  const int maxbv = f32 ? 32 : 64;
  int bv = Dv < maxbv ? Dv : maxbv;
  while (bv > 16 && (long)B * H * (Dv / bv) < 256) bv /= 2;
  return bv;
}

template <int DK, int C, bool F32IN>
static hipError_t launch_fwd_bv(const FwdArgs& a, hipStream_t s) {
  switch (pick_bv(a.B, a.H, a.Dv, F32IN)) {
    case 16: return launch_fwd_t<DK, C, 16, F32IN>(a, s);
    case 32: return launch_fwd_t<DK, C, 32, F32IN>(a, s);
    case 64:
      if constexpr (F32IN) return hipErrorInvalidValue;
      else return launch_fwd_t<DK, C, 64, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DK, bool F32IN>
static hipError_t launch_fwd_c(const FwdArgs& a, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_fwd_bv<DK, 16, F32IN>(a, s);
    case 32: return launch_fwd_bv<DK, 32, F32IN>(a, s);
    case 64: return launch_fwd_bv<DK, 64, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_fwd_dk(const FwdArgs& a, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_fwd_c<16, F32IN>(a, s);
    case 32: return launch_fwd_c<32, F32IN>(a, s);
    case 64: return launch_fwd_c<64, F32IN>(a, s);
    case 128: return launch_fwd_c<128, F32IN>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.f32_inputs ? launch_fwd_dk<true>(a, stream) : launch_fwd_dk<false>(a, stream);
}

template <int DK, int C, bool F32IN>
static bool fits_all_bv() {
  return FwdCfg<DK, C, 16, F32IN>::kFits && FwdCfg<DK, C, 32, F32IN>::kFits &&
         (F32IN || FwdCfg<DK, C, 64, F32IN>::kFits);
}

template <int DK, bool F32IN>
static bool fwd_fits_c(int chunk) {
  switch (chunk) {
    case 16: return fits_all_bv<DK, 16, F32IN>();
    case 32: return fits_all_bv<DK, 32, F32IN>();
    case 64: return fits_all_bv<DK, 64, F32IN>();
  }
  return false;
}

template <bool F32IN>
static bool fwd_fits(int Dk, int chunk) {
  switch (Dk) {
    case 16: return fwd_fits_c<16, F32IN>(chunk);
    case 32: return fwd_fits_c<32, F32IN>(chunk);
    case 64: return fwd_fits_c<64, F32IN>(chunk);
    case 128: return fwd_fits_c<128, F32IN>(chunk);
  }
  return false;
}

bool fwd_supported(int Dk, int Dv, int chunk, bool f32_inputs) {
  (void)Dv;
  return f32_inputs ? fwd_fits<true>(Dk, chunk) : fwd_fits<false>(Dk, chunk);
}

}  // namespace gdn2
