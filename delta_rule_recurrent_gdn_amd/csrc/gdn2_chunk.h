// gdn2_chunk.h -- per-chunk key-side preparation shared by the forward and the
// backward kernels of the Gated Delta Rule-2 operator.
//
// For one chunk of C tokens of one (batch, head) this computes, inside one
// workgroup of NT threads (chunkwise WY algorithm with the channel-wise decay
// absorbed into asymmetric erase factors; arXiv 2605.22791 abstract):
//
//   g      in-chunk inclusive cumulative sum of log_alpha      (gate preprocessing)
//   A      strict_lower(Kh' Kt'^T),  Kh' = b*k*exp(g - g_m),  Kt' = k*exp(g_m - g)
//   P      lower_incl(Qh' Kt'^T),    Qh' = q*exp(g - g_m)
//   T      (I + A)^-1
//
// where g_m is g at the middle of the chunk: the pairs exp(+-(g - g_m)) only
// span half a chunk of decay, and their products exp(g_r - g_i) (i <= r) are
// exactly the decay between two tokens. A and P are formed from a two-term
// bf16 split of these wide-range operands (fp32 operands for fp32 inputs).
// The caller receives, per element, q, k, b and the decay factors through a
// "sink" so that it can write whichever chunk-start-referenced operands it
// needs (b*k*exp(g), q*exp(g), k*exp(g_C - g), ...).
//
// Raw inputs of the next chunk are fetched into registers by load() while the
// current chunk is still being processed.
#pragma once

#include <type_traits>

#include "gdn2_common.h"
#include "gdn2_wide.h"

namespace gdn2 {

// lower-triangular tile index p -> (R, I) with I <= R, R-major
__device__ __forceinline__ void tri_index(int p, int& R, int& I) {
  R = 0;
  while (p > R) {
    p -= R + 1;
    ++R;
  }
  I = p;
}

// N (1 or 4) consecutive fp32 values to / from LDS in one access
template <int N>
__device__ __forceinline__ void st_lanes(float* dst, const float (&x)[N]) {
  if constexpr (N == 4) *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
  else *dst = x[0];
}
template <int N>
__device__ __forceinline__ void ld_lanes(float (&x)[N], const float* src) {
  if constexpr (N == 4) {
    const float4 v = *reinterpret_cast<const float4*>(src);
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  } else {
    x[0] = *src;
  }
}

template <int DK, int C, bool F32IN, int NT = 512, int LAW = 1>
struct KSide {
  using OpT = typename std::conditional<F32IN, float, _Float16>::type;  // value-side operand type
  static constexpr int NW = NT / kWave;
  static constexpr int NB = C / 16;                   // 16-token row blocks
  static constexpr int SW = DK < 32 ? DK : 32;        // channel slice of the Gram phase
  static constexpr int NSL = DK / SW;
  static constexpr int PADOP = F32IN ? 4 : 8;         // 16-byte row padding
  static constexpr int LDC = C + PADOP;               // operand rows of C tokens
  static constexpr int LDK = DK + PADOP;              // operand rows of DK channels
  static constexpr int LDSW = SW + (F32IN ? 4 : 8);   // Gram slice rows
  static constexpr int LDCF = C + 4;                  // fp32 [C][C]
  static constexpr int LDX = 20;                      // fp32 16x16 scratch tiles
  // log_alpha: each thread owns LAW adjacent channels (1 or 4) of LA_RPS consecutive rows.
  // The wide form takes fewer instructions; the narrow one fewer address registers.
  static_assert(LAW == 1 || LAW == 4, "log_alpha vector width");
  static constexpr int LA_SEGS = (NT / (DK / LAW)) < C ? (NT / (DK / LAW)) : C;
  static constexpr int LA_RPS = C / LA_SEGS;
  // q, k, b: groups of 4 channels of one row; rows qk_r + i * QK_RPP, i < QK_RPT
  static constexpr int QK_RPP = NT / (SW / 4);
  static constexpr int QK_RPT = (C + QK_RPP - 1) / QK_RPP;
  static constexpr int GRAMB = F32IN ? 4 : 2;
  static constexpr int GRAMPARTS = F32IN ? 3 : 6;     // Kh', Qh', Kt' (hi/lo each for the bf16 split)
  static constexpr int kSliceBytes = C * LDSW * GRAMB;
  static constexpr int NGT = NB * (NB + 1);           // lower tiles of A and of P
  static constexpr int GPW = (NGT + NW - 1) / NW;

  // LDS byte sizes of the pieces used here
  static constexpr int kGBytes = C * DK * 4;               // g [C][DK]
  static constexpr int kSlicesBytes = GRAMPARTS * kSliceBytes;
  static constexpr int kChanBytes = 4 * DK * 4;            // g_m, g_C, exp(g_m), exp(g_C - g_m)
  static constexpr int kTotBytes = LA_SEGS * DK * 4;       // cumsum segment totals
  static constexpr int kAfBytes = C * LDCF * 4;            // A, then T (fp32)
  static constexpr int kXsBytes = 4 * 16 * LDX * 4;        // inversion scratch
  static_assert(LA_SEGS >= 2 && LA_SEGS * LA_RPS == C, "cumsum tiling");

  // ---- raw registers of one chunk ----
  float la[LA_RPS][LAW];
  Raw4<F32IN> rq[NSL][QK_RPT], rk[NSL][QK_RPT], rb[NSL][QK_RPT];
  int la_c, la_sg, qk_r, qk_c4;
  bool la_on, qk_on;
  bool raw = false;  // pre-activation gates: log_alpha = -softplus(input), b = sigmoid(input)
  bool scalar_la = false, scalar_b = false;  // one value per (token, head), [., T, H], broadcast

  __device__ __forceinline__ void init(int tid) {
    la_c = LAW * (tid % (DK / LAW));  // first of the thread's channels
    la_sg = tid / (DK / LAW);
    la_on = la_sg < LA_SEGS;
    qk_r = tid / (SW / 4);
    qk_c4 = tid % (SW / 4);
    qk_on = qk_r < C && qk_r < QK_RPP;
  }

  // Fetch only the log_alpha rows of the chunk (for gates()).
  __device__ __forceinline__ void load_la(const float* log_alpha, int64_t baseK, int64_t rowK, int tn, int Ln) {
    if (la_on) {
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i) {
        const int r = la_sg * LA_RPS + i;
        const int64_t idx = baseK + (int64_t)(tn + r) * rowK + la_c;
        const int64_t sidx = baseK / DK + (int64_t)(tn + r) * (rowK / DK);
        if constexpr (LAW == 4) {
          const float4 x = r < Ln ? load_la4(log_alpha, idx, sidx, scalar_la) : make_float4(0.f, 0.f, 0.f, 0.f);
          la[i][0] = x.x;
          la[i][1] = x.y;
          la[i][2] = x.z;
          la[i][3] = x.w;
        } else {
          la[i][0] = r < Ln ? log_alpha[scalar_la ? sidx : idx] : 0.f;
        }
      }
      if (raw) {
#pragma unroll
        for (int i = 0; i < LA_RPS; ++i)
#pragma unroll
          for (int j = 0; j < LAW; ++j)
            if (la_sg * LA_RPS + i < Ln) la[i][j] = neg_softplus_f(la[i][j]);  // padding rows stay 0
      }
    }
  }

  // Fetch chunk rows [tn, tn + Ln) of one (batch, head): base* index token 0.
  __device__ __forceinline__ void load(const void* q, const void* k, const void* b, const float* log_alpha,
                                      int64_t baseK, int64_t rowK, int tn, int Ln) {
    if (la_on) {
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i) {
        const int r = la_sg * LA_RPS + i;
        const int64_t idx = baseK + (int64_t)(tn + r) * rowK + la_c;
        const int64_t sidx = baseK / DK + (int64_t)(tn + r) * (rowK / DK);
        if constexpr (LAW == 4) {
          const float4 x = r < Ln ? load_la4(log_alpha, idx, sidx, scalar_la) : make_float4(0.f, 0.f, 0.f, 0.f);
          la[i][0] = x.x;
          la[i][1] = x.y;
          la[i][2] = x.z;
          la[i][3] = x.w;
        } else {
          la[i][0] = r < Ln ? log_alpha[scalar_la ? sidx : idx] : 0.f;
        }
      }
      if (raw) {
#pragma unroll
        for (int i = 0; i < LA_RPS; ++i)
#pragma unroll
          for (int j = 0; j < LAW; ++j)
            if (la_sg * LA_RPS + i < Ln) la[i][j] = neg_softplus_f(la[i][j]);  // padding rows stay 0
      }
    }
    if (qk_on) {
#pragma unroll
      for (int s = 0; s < NSL; ++s) {
#pragma unroll
        for (int i = 0; i < QK_RPT; ++i) {
          const int r = qk_r + i * QK_RPP;
          if (r < Ln) {
            const int64_t idx = baseK + (int64_t)(tn + r) * rowK + s * SW + 4 * qk_c4;
            ld_raw(rq[s][i], q, idx);
            ld_raw(rk[s][i], k, idx);
            ld_raw_gate(rb[s][i], b, idx, baseK / DK + (int64_t)(tn + r) * (rowK / DK), scalar_b);
          } else {
            zero_raw(rq[s][i]);
            zero_raw(rk[s][i]);
            zero_raw(rb[s][i]);
          }
        }
      }
    }
  }

  // Gate preprocessing: g (sG, fp32 [C][DK]) and the per-channel constants in
  // sChan = {g_m, g_C, exp(g_m), exp(g_C - g_m)} (each [DK]). The caller must
  // have synchronised since the last readers of sG/sChan/sTot. Ends synchronised.
  // Returns (in every thread) whether the chunk is a wide-decay one: on some
  // channel |g - g_m| exceeds kWideSpan (gdn2_wide.h).
  __device__ __forceinline__ bool gates(float* sTot, float* sG, float* sChan) {
    bool far = false;
    if (la_on) {
      float run[LAW];
#pragma unroll
      for (int j = 0; j < LAW; ++j) run[j] = 0.f;
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i)
#pragma unroll
        for (int j = 0; j < LAW; ++j) {
          run[j] += la_floor(la[i][j]);  // per-token log-decay floor (gdn2_wide.h)
          la[i][j] = run[j];
        }
      st_lanes(sTot + la_sg * DK + la_c, run);
    }
    __syncthreads();
    if (la_on) {
      float off[LAW], gmid[LAW], gend[LAW];
#pragma unroll
      for (int j = 0; j < LAW; ++j) off[j] = gmid[j] = gend[j] = 0.f;
#pragma unroll
      for (int sgi = 0; sgi < LA_SEGS; ++sgi) {
        float tt[LAW];
        ld_lanes(tt, sTot + sgi * DK + la_c);
#pragma unroll
        for (int j = 0; j < LAW; ++j) {
          if (sgi < la_sg) off[j] += tt[j];
          if (sgi < LA_SEGS / 2) gmid[j] += tt[j];  // the middle row C/2-1 ends segment LA_SEGS/2-1
          gend[j] += tt[j];
        }
      }
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i) {
        float g[LAW];
#pragma unroll
        for (int j = 0; j < LAW; ++j) {
          g[j] = la[i][j] + off[j];
          far = far || fabsf(g[j] - gmid[j]) > kWideSpan;
        }
        st_lanes(sG + (la_sg * LA_RPS + i) * DK + la_c, g);
      }
      if (la_sg == 0) {
        float e1[LAW], e2[LAW];
#pragma unroll
        for (int j = 0; j < LAW; ++j) {
          e1[j] = __expf(gmid[j]);
          e2[j] = __expf(gend[j] - gmid[j]);
        }
        st_lanes(sChan + la_c, gmid);
        st_lanes(sChan + DK + la_c, gend);
        st_lanes(sChan + 2 * DK + la_c, e1);
        st_lanes(sChan + 3 * DK + la_c, e2);
      }
    }
    return __builtin_amdgcn_readfirstlane(__syncthreads_or(far)) != 0;  // uniform: a scalar branch
  }

  // Wide-decay chunks (gdn2_wide.h): from log_alpha rows fetched again by
  // load_la(), the cumulative log-decay from the start of each row's 16-token
  // block into sG (fp32 [C][DK]), the block totals into sBs [NB][DK] and the
  // pair scales into sPS. Same synchronisation contract as gates().
  __device__ __forceinline__ void gates_block(float* sTot, float* sG, float* sBs, float* sPS) {
    constexpr int SPB = 16 / LA_RPS;  // cumsum segments per 16-token block
    static_assert(LA_RPS <= 16 && 16 % LA_RPS == 0, "segments tile the blocks");
    if (la_on) {
      float run[LAW];
#pragma unroll
      for (int j = 0; j < LAW; ++j) run[j] = 0.f;
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i)
#pragma unroll
        for (int j = 0; j < LAW; ++j) {
          run[j] += la_floor(la[i][j]);
          la[i][j] = run[j];
        }
      st_lanes(sTot + la_sg * DK + la_c, run);
    }
    __syncthreads();
    if (la_on) {
      float off[LAW];
#pragma unroll
      for (int j = 0; j < LAW; ++j) off[j] = 0.f;
      for (int sgi = (la_sg / SPB) * SPB; sgi < la_sg; ++sgi) {
        float tt[LAW];
        ld_lanes(tt, sTot + sgi * DK + la_c);
#pragma unroll
        for (int j = 0; j < LAW; ++j) off[j] += tt[j];
      }
#pragma unroll
      for (int i = 0; i < LA_RPS; ++i) {
        float g[LAW];
#pragma unroll
        for (int j = 0; j < LAW; ++j) g[j] = la[i][j] + off[j];
        st_lanes(sG + (la_sg * LA_RPS + i) * DK + la_c, g);
        if (la_sg % SPB == SPB - 1 && i == LA_RPS - 1) st_lanes(sBs + (la_sg / SPB) * DK + la_c, g);
      }
    }
    __syncthreads();
    wide_pair_scales<NB, DK, NT>(sBs, sPS);
    __syncthreads();
  }

  // Factor pass and Gram products. For each channel slice: every thread turns
  // its 4 (row, channel) inputs into the Gram factors (LDS slices) and hands
  // q, k, b, e1 = exp(g - g_m), eg = exp(g), ec = exp(g_C - g) to sink(r, c0, ...),
  // then A and P accumulate over the slice. Ends synchronised; on return accG
  // holds the lower tiles of A (first NGT/2 tile indices) and P (the rest).
  template <class Sink>
  __device__ __forceinline__ void factors_gram(const float* sG, const float* sChan, char* sSL,
                                               f32x4 (&accG)[GPW], Sink&& sink) {
    const int wid = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < GPW; ++i) accG[i] = zero4();
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
      for (int ri = 0; ri < QK_RPT; ++ri) {
        const int r = qk_r + ri * QK_RPP, cl = 4 * qk_c4, c0 = sl * SW + cl;
        if (!qk_on || r >= C) continue;
        float qv[4], kv[4], bv[4];
        cvt(rq[sl][ri], qv);
        cvt(rk[sl][ri], kv);
        cvt(rb[sl][ri], bv);
        if (raw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) bv[i] = sigmoid_f(bv[i]);  // k is zero on padding rows
        }
        const float4 g4 = *reinterpret_cast<const float4*>(sG + r * DK + c0);
        const float4 gm4 = *reinterpret_cast<const float4*>(sChan + c0);
        const float4 eg4 = *reinterpret_cast<const float4*>(sChan + 2 * DK + c0);
        const float4 ec4 = *reinterpret_cast<const float4*>(sChan + 3 * DK + c0);
        const float gg[4] = {g4.x, g4.y, g4.z, g4.w}, gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
        const float egm[4] = {eg4.x, eg4.y, eg4.z, eg4.w}, egcm[4] = {ec4.x, ec4.y, ec4.z, ec4.w};
        float e1[4], eg[4], ec[4], khm[4], qhm[4], ktm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e1[i] = __expf(gg[i] - gm[i]);                 // exp(g - g_m)
          const float e2 = __builtin_amdgcn_rcpf(e1[i]);  // exp(g_m - g)
          eg[i] = e1[i] * egm[i];                        // exp(g)
          ec[i] = egcm[i] * e2;                          // exp(g_C - g)
          khm[i] = bv[i] * kv[i] * e1[i];
          qhm[i] = qv[i] * e1[i];
          ktm[i] = kv[i] * e2;
        }
        if constexpr (F32IN) {
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
        sink(r, c0, qv, kv, bv, e1, eg, ec);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int t = wid + NW * i;
        if (t < NGT) {
          const bool isP = t >= NGT / 2;
          int R, I;
          tri_index(isP ? t - NGT / 2 : t, R, I);
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
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    }
  }

  // A -> sAf (fp32, strict lower, zero above); P -> sP (operand type, lower incl.
  // diagonal, zero above), row-major when PT is false, transposed when true.
  template <bool PT>
  __device__ __forceinline__ void gram_store(const f32x4 (&accG)[GPW], float* sAf, OpT* sP) {
    const int wid = threadIdx.x / kWave, l = lane_id(), lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int t = wid + NW * i;
      if (t < NGT) {
        const bool isP = t >= NGT / 2;
        int R, I;
        tri_index(isP ? t - NGT / 2 : t, R, I);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * R + 4 * lg + e, col = 16 * I + lr;
          if (isP) {
            const OpT v = static_cast<OpT>(row >= col ? accG[i][e] : 0.f);
            if (PT) sP[col * LDC + row] = v;
            else sP[row * LDC + col] = v;
          } else {
            sAf[row * LDCF + col] = row > col ? accG[i][e] : 0.f;
          }
        }
      }
    }
    // P's upper blocks (I > R) are never written above: clear them so that
    // products over the full chunk length see zeros there
    for (int e = threadIdx.x; e < C * C; e += NT) {
      const int row = e / C, col = e % C;
      if ((col >> 4) > (row >> 4)) {
        if (PT) sP[col * LDC + row] = static_cast<OpT>(0.f);
        else sP[row * LDC + col] = static_cast<OpT>(0.f);
      }
    }
  }

  // T = (I + A)^-1 in place in sAf (fp32): 16x16 diagonal blocks by one wave
  // each, then the off-diagonal blocks by block products,
  //   T_{IJ} = -T_{II} (sum_{K=J}^{I-1} A_{IK} T_{KJ}),
  // in two levels (16 -> 32 -> 64 rows). Begins and ends with a barrier.
  __device__ __forceinline__ void invert(float* sAf, float* sXs) {
    const int wid = threadIdx.x / kWave;
    __syncthreads();
    if (wid < NB) invert_unit_lower16<OpT>(sAf + 16 * wid * LDCF + 16 * wid, LDCF);
    __syncthreads();
    if constexpr (NB >= 2) {
      if (wid < NB / 2) {
        const int I = 2 * wid + 1, J = 2 * wid;
        f32x4 x = zero4();
        mma_f32src<OpT, false>(x, sAf + 16 * I * LDCF + 16 * J, LDCF, sAf + 16 * J * LDCF + 16 * J, LDCF, 16);
        store_tile(sXs + wid * 16 * LDX, LDX, x);
      }
      __syncthreads();
      if (wid < NB / 2) {
        const int I = 2 * wid + 1, J = 2 * wid;
        f32x4 y = zero4();
        mma_f32src<OpT, false>(y, sAf + 16 * I * LDCF + 16 * I, LDCF, sXs + wid * 16 * LDX, LDX, 16);
        store_tile(sAf + 16 * I * LDCF + 16 * J, LDCF, y, -1.f);
      }
      __syncthreads();
    }
    if constexpr (NB == 4) {
      if (wid < 4) {
        const int I = 2 + wid / 2, J = wid % 2;
        f32x4 x = zero4();
        for (int K = J; K <= 1; ++K)
          mma_f32src<OpT, false>(x, sAf + 16 * I * LDCF + 16 * K, LDCF, sAf + 16 * K * LDCF + 16 * J, LDCF, 16);
        store_tile(sXs + wid * 16 * LDX, LDX, x);
      }
      __syncthreads();
      if (wid < 4) {
        const int I = 2 + wid / 2, J = wid % 2;
        f32x4 y = zero4();
        for (int K = 2; K <= I; ++K)
          mma_f32src<OpT, false>(y, sAf + 16 * I * LDCF + 16 * K, LDCF, sXs + ((K - 2) * 2 + J) * 16 * LDX, LDX,
                                 16);
        store_tile(sAf + 16 * I * LDCF + 16 * J, LDCF, y, -1.f);
      }
      __syncthreads();
    }
    // blocks above the diagonal of T are zero
    for (int e = threadIdx.x; e < C * C; e += NT) {
      const int row = e / C, col = e % C;
      if ((col >> 4) > (row >> 4)) sAf[row * LDCF + col] = 0.f;
    }
    __syncthreads();
  }
};

}  // namespace gdn2
