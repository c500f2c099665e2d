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

#include <type_traits>

#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <int DK, int C, int BV, bool F32IN>
struct FwdCfg {
  using OpT = typename std::conditional<F32IN, float, _Float16>::type;  // value-side operand type
  using TriT = OpT;                                                     // operand type of the T blocks
  static constexpr int kThreads = 256;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int NB = C / 16;                    // 16-token row blocks per chunk
  static constexpr int SW = DK < 32 ? DK : 32;         // channel slice of the Gram phase
  static constexpr int NSL = DK / SW;
  static constexpr int PADOP = F32IN ? 4 : 8;          // 16-byte row padding
  static constexpr int LDC = C + PADOP;                // rows of C tokens
  static constexpr int LDK = DK + PADOP;               // rows of DK channels
  static constexpr int LDSW = SW + (F32IN ? 4 : 8);    // Gram slice rows
  static constexpr int LDCF = C + 4;                   // fp32 [C][C] (A, then T)
  static constexpr int LDX = 20;                       // fp32 16x16 scratch tiles
  static constexpr int OPB = sizeof(OpT);
  static constexpr int GRAMB = F32IN ? 4 : 2;          // bytes per Gram slice element (per part)
  static constexpr int GRAMPARTS = F32IN ? 3 : 6;      // KhM, QhM, KtM (hi/lo each for bf16 split)

  // persistent region
  static constexpr int oKhT = 0;                                   // OpT [DK][LDC]
  static constexpr int oQs = oKhT + DK * LDC * OPB;                // OpT [C][LDK]
  static constexpr int oKbT = oQs + C * LDK * OPB;                 // OpT [DK][LDC]
  static constexpr int oWVT = oKbT + DK * LDC * OPB;               // OpT [BV][LDC]
  static constexpr int oST = oWVT + BV * LDC * OPB;                // OpT [BV][LDK]
  static constexpr int oGC = oST + BV * LDK * OPB;                 // float [DK]
  static constexpr int oGM = oGC + DK * 4;                         // float [DK]
  static constexpr int oX = oGM + DK * 4;                          // start of the phase-shared region
  // phase F (gate preprocessing + Gram)
  static constexpr int oG = oX;                                    // float [C][DK]
  static constexpr int oSL = oG + C * DK * 4;                      // Gram slices
  static constexpr int kSliceBytes = C * LDSW * GRAMB;
  static constexpr int endF = oSL + GRAMPARTS * kSliceBytes;
  // phase W (after the Gram products)
  static constexpr int oAf = oX;                                   // float [C][LDCF]
  static constexpr int oPm = oAf + C * LDCF * 4;                   // OpT [C][LDC]
  static constexpr int oWm = oPm + C * LDC * OPB;                  // OpT [C][LDK]  (holds -W)
  static constexpr int oUT = oWm + C * LDK * OPB;                  // OpT [BV][LDC]
  static constexpr int oXs = oUT + BV * LDC * OPB;                 // float [4][16][LDX]
  static constexpr int endW = oXs + 4 * 16 * LDX * 4;
  static constexpr int kLdsBytes = endF > endW ? endF : endW;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;

  static constexpr int NGT = NB * (NB + 1);                        // A and P lower tiles
  static constexpr int GPW = (NGT + kWaves - 1) / kWaves;
  static constexpr int NUT = NB * (BV / 16);                       // U / O tiles
  static constexpr int UPW = (NUT + kWaves - 1) / kWaves;
  static constexpr int NST = (DK / 16) * (BV / 16);                // state tiles
  static constexpr int SPW = (NST + kWaves - 1) / kWaves;
  static constexpr int NWT = (DK / 16) * NB;                       // W^T tiles
  static constexpr int WPW = (NWT + kWaves - 1) / kWaves;
};

// lower-triangular tile index p -> (R, I) with I <= R, R-major
__device__ __forceinline__ void tri_index(int p, int& R, int& I) {
  R = 0;
  while (p > R) {
    p -= R + 1;
    ++R;
  }
  I = p;
}

template <int DK, int C, int BV, bool F32IN>
__global__ __launch_bounds__(256) void gdn2_fwd_kernel(FwdArgs a) {
  using Cfg = FwdCfg<DK, C, BV, F32IN>;
  using OpT = typename Cfg::OpT;
  using TriT = typename Cfg::TriT;
  constexpr int NW = Cfg::kWaves, NT = Cfg::kThreads, NB = Cfg::NB, SW = Cfg::SW;
  constexpr int LDC = Cfg::LDC, LDK = Cfg::LDK, LDSW = Cfg::LDSW, LDCF = Cfg::LDCF, LDX = Cfg::LDX;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  OpT* sKhT = reinterpret_cast<OpT*>(smem + Cfg::oKhT);
  OpT* sQs = reinterpret_cast<OpT*>(smem + Cfg::oQs);
  OpT* sKbT = reinterpret_cast<OpT*>(smem + Cfg::oKbT);
  OpT* sWVT = reinterpret_cast<OpT*>(smem + Cfg::oWVT);
  OpT* sST = reinterpret_cast<OpT*>(smem + Cfg::oST);
  float* sgC = reinterpret_cast<float*>(smem + Cfg::oGC);
  float* sgm = reinterpret_cast<float*>(smem + Cfg::oGM);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* sSL = smem + Cfg::oSL;
  float* sAf = reinterpret_cast<float*>(smem + Cfg::oAf);
  OpT* sPm = reinterpret_cast<OpT*>(smem + Cfg::oPm);
  OpT* sWm = reinterpret_cast<OpT*>(smem + Cfg::oWm);
  OpT* sUT = reinterpret_cast<OpT*>(smem + Cfg::oUT);
  float* sXs = reinterpret_cast<float*>(smem + Cfg::oXs);

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
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

  for (int n = 0; n < NC; ++n) {
    const int t0 = n * C;
    const int Lr = min(C, T - t0);

    if (a.chunk_states) {
      float* cs = a.chunk_states + ((int64_t)bh * NC + n) * DK * Dv + j0;
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

    // ---- (1) gate preprocessing: log_alpha -> sG, w*v -> sWVT ----
    for (int e = tid; e < C * (DK / 4); e += NT) {
      const int r = e / (DK / 4), c4 = e % (DK / 4);
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < Lr) val = *reinterpret_cast<const float4*>(a.log_alpha + baseK + (int64_t)(t0 + r) * rowK + 4 * c4);
      *reinterpret_cast<float4*>(sG + r * DK + 4 * c4) = val;
    }
    for (int e = tid; e < C * (BV / 8); e += NT) {
      const int r = e / (BV / 8), j8 = e % (BV / 8);
      float vv[8], ww[8];
      if (r < Lr) {
        load8<F32IN>(a.v, baseV + (int64_t)(t0 + r) * rowV + 8 * j8, vv);
        load8<F32IN>(a.w, baseV + (int64_t)(t0 + r) * rowV + 8 * j8, ww);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = ww[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sWVT[(8 * j8 + i) * LDC + r] = static_cast<OpT>(ww[i] * vv[i]);
    }
    __syncthreads();
    for (int c = tid; c < DK; c += NT) {
      float run = 0.f;
#pragma unroll 16
      for (int r = 0; r < C; ++r) {
        run += sG[r * DK + c];
        sG[r * DK + c] = run;
        if (r == C / 2 - 1) sgm[c] = run;
      }
      sgC[c] = run;
    }
    __syncthreads();

    // ---- (2)+(3a) factors and the Gram products A, P (channel slices) ----
    f32x4 accG[Cfg::GPW];
#pragma unroll
    for (int i = 0; i < Cfg::GPW; ++i) accG[i] = zero4();

    for (int sl = 0; sl < Cfg::NSL; ++sl) {
      for (int e = tid; e < C * (SW / 8); e += NT) {
        const int r = e / (SW / 8), cl = 8 * (e % (SW / 8));
        const int c0 = sl * SW + cl;
        float qv[8], kv[8], bv[8];
        if (r < Lr) {
          const int64_t idx = baseK + (int64_t)(t0 + r) * rowK + c0;
          load8<F32IN>(a.q, idx, qv);
          load8<F32IN>(a.k, idx, kv);
          load8<F32IN>(a.b, idx, bv);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) qv[i] = kv[i] = bv[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = c0 + i;
          const float g = sG[r * DK + c], gm = sgm[c], gc = sgC[c];
          const float eg = __expf(g), emr = __expf(g - gm), emc = __expf(gm - g), ec = __expf(gc - g);
          const float bk = bv[i] * kv[i];
          const float khm = bk * emr, qhm = qv[i] * emr, ktm = kv[i] * emc;
          if constexpr (F32IN) {
            float* sl0 = reinterpret_cast<float*>(sSL);
            sl0[0 * (C * LDSW) + r * LDSW + cl + i] = khm;
            sl0[1 * (C * LDSW) + r * LDSW + cl + i] = qhm;
            sl0[2 * (C * LDSW) + r * LDSW + cl + i] = ktm;
          } else {
            __bf16* sl0 = reinterpret_cast<__bf16*>(sSL);
            const __bf16 kh_h = f32_to_bf16(khm), qh_h = f32_to_bf16(qhm), kt_h = f32_to_bf16(ktm);
            const int o = r * LDSW + cl + i;
            sl0[0 * (C * LDSW) + o] = kh_h;
            sl0[1 * (C * LDSW) + o] = f32_to_bf16(khm - bf16_to_f32(kh_h));
            sl0[2 * (C * LDSW) + o] = qh_h;
            sl0[3 * (C * LDSW) + o] = f32_to_bf16(qhm - bf16_to_f32(qh_h));
            sl0[4 * (C * LDSW) + o] = kt_h;
            sl0[5 * (C * LDSW) + o] = f32_to_bf16(ktm - bf16_to_f32(kt_h));
          }
          sKhT[c * LDC + r] = static_cast<OpT>(bk * eg);
          sQs[r * LDK + c] = static_cast<OpT>(qv[i] * eg);
          sKbT[c * LDC + r] = static_cast<OpT>(kv[i] * ec);
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < Cfg::GPW; ++i) {
        const int t = wid + NW * i;
        if (t < Cfg::NGT) {
          const bool isP = t >= Cfg::NGT / 2;
          int R, I;
          tri_index(isP ? t - Cfg::NGT / 2 : t, R, I);
          if constexpr (F32IN) {
            const float* sl0 = reinterpret_cast<const float*>(sSL);
            const float* X = sl0 + (isP ? 1 : 0) * (C * LDSW) + 16 * R * LDSW;
            const float* Y = sl0 + 2 * (C * LDSW) + 16 * I * LDSW;
            mma_nt_k<SW>(accG[i], X, LDSW, Y, LDSW);
          } else {
            const __bf16* sl0 = reinterpret_cast<const __bf16*>(sSL);
            const __bf16* Xh = sl0 + (isP ? 2 : 0) * (C * LDSW) + 16 * R * LDSW;
            const __bf16* Y0 = sl0 + 4 * (C * LDSW) + 16 * I * LDSW;
            mma_nt_split_k<SW>(accG[i], Xh, Xh + C * LDSW, LDSW, Y0, Y0 + C * LDSW, LDSW);
          }
        }
      }
      __syncthreads();
    }

    // ---- A -> sAf (strict lower), P -> sPm (lower incl. diagonal) ----
#pragma unroll
    for (int i = 0; i < Cfg::GPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NGT) {
        const bool isP = t >= Cfg::NGT / 2;
        int R, I;
        tri_index(isP ? t - Cfg::NGT / 2 : t, R, I);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
          if (isP) sPm[row * LDC + col] = static_cast<OpT>(row >= col ? accG[i][e] : 0.f);
          else sAf[row * LDCF + col] = row > col ? accG[i][e] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- (3b) T = (I + A)^-1: diagonal 16x16 blocks by forward substitution ----
    if (wid < NB && l < 16) {
      float* Ab = sAf + 16 * wid * LDCF + 16 * wid;
      float tcol[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) tcol[m] = (m == l) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s += Ab[r * LDCF + m] * tcol[m];
        if (r > l) tcol[r] = -s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Ab[r * LDCF + l] = tcol[r];
    }
    __syncthreads();
    // level 1: T_{2j+1,2j} = -T_{2j+1,2j+1} A_{2j+1,2j} T_{2j,2j}
    if constexpr (NB >= 2) {
      if (wid < NB / 2) {
        const int I = 2 * wid + 1, J = 2 * wid;
        f32x4 x = zero4();
        mma_f32src<TriT, false>(x, sAf + 16 * I * LDCF + 16 * J, LDCF, sAf + 16 * J * LDCF + 16 * J, LDCF, 16);
        store_tile(sXs + wid * 16 * LDX, LDX, x);
      }
      __syncthreads();
      if (wid < NB / 2) {
        const int I = 2 * wid + 1, J = 2 * wid;
        f32x4 y = zero4();
        mma_f32src<TriT, false>(y, sAf + 16 * I * LDCF + 16 * I, LDCF, sXs + wid * 16 * LDX, LDX, 16);
        store_tile(sAf + 16 * I * LDCF + 16 * J, LDCF, y, -1.f);
      }
      __syncthreads();
    }
    // level 2 (C = 64): T_{[23],[01]} = -T_{[23],[23]} A_{[23],[01]} T_{[01],[01]}
    if constexpr (NB == 4) {
      {
        const int I = 2 + wid / 2, J = wid % 2;
        f32x4 x = zero4();
        for (int K = J; K <= 1; ++K)
          mma_f32src<TriT, false>(x, sAf + 16 * I * LDCF + 16 * K, LDCF, sAf + 16 * K * LDCF + 16 * J, LDCF, 16);
        store_tile(sXs + wid * 16 * LDX, LDX, x);
      }
      __syncthreads();
      {
        const int I = 2 + wid / 2, J = wid % 2;
        f32x4 y = zero4();
        for (int K = 2; K <= I; ++K)
          mma_f32src<TriT, false>(y, sAf + 16 * I * LDCF + 16 * K, LDCF, sXs + ((K - 2) * 2 + J) * 16 * LDX, LDX, 16);
        store_tile(sAf + 16 * I * LDCF + 16 * J, LDCF, y, -1.f);
      }
      __syncthreads();
    }

    // ---- (4a) W^T = Kh^T T^T -> sWm holds -W ; U tiles start as T (w*v) ----
#pragma unroll
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
      }
    }
    __syncthreads();

    // ---- (4b) U = T(w*v) - W S ; O = (q*exp(g)) S ----
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NUT) {
        const int R = t / (BV / 16), jb = t % (BV / 16);
        mma_nt_k<DK>(accU[i], sWm + 16 * R * LDK, LDK, sST + 16 * jb * LDK, LDK);
        mma_nt_k<DK>(accO[i], sQs + 16 * R * LDK, LDK, sST + 16 * jb * LDK, LDK);
        store_tile_t(sUT + 16 * jb * LDC + 16 * R, LDC, accU[i]);
      }
    }
    __syncthreads();

    // ---- (4c) O += P U -> o ;  S <- Diag(exp(g_C)) S + Kb^T U ----
#pragma unroll
    for (int i = 0; i < Cfg::UPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NUT) {
        const int R = t / (BV / 16), jb = t % (BV / 16);
        if (a.o == nullptr) continue;  // state-only pass (chunk states for the backward)
        mma_nt<OpT>(accO[i], sPm + 16 * R * LDC, LDC, sUT + 16 * jb * LDC, LDC, 16 * (R + 1));
        float* op = a.o + baseV + 16 * jb + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          if (r < Lr) op[(int64_t)(t0 + r) * rowV] = accO[i][e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
      const int t = wid + NW * i;
      if (t < Cfg::NST) {
        const int cb = t / (BV / 16), jb = t % (BV / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= __expf(sgC[16 * cb + 4 * lg + e]);
        mma_nt_k<C>(accS[i], sKbT + 16 * cb * LDC, LDC, sUT + 16 * jb * LDC, LDC);
        store_tile_t(sST + 16 * jb * LDK + 16 * cb, LDK, accS[i]);
      }
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
    hipLaunchKernelGGL((gdn2_fwd_kernel<DK, C, BV, F32IN>), dim3(grid), dim3(256), 0, stream, a);
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
