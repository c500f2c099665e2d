// gdn2_chain.hip -- sequential half of the two-stage chunkwise forward: the
// state-dependent part of every chunk, in chunk order.
//
// With the per-chunk record written by the preparation kernel (-W, Qs = q exp(g),
// Kb^T, P, gamma = exp(g_C) and Ut = T (w v)), a chunk entered with state S
// (Dk x Dv, fp32) needs (arXiv 2605.22791 abstract; research-wiki summary,
// "Key findings": the chunkwise WY refactoring of the recurrence)
//   U = Ut - W S,   O = Qs S + P U,   S <- Diag(gamma) S + Kb^T U.
// Every operator acts on S from the left, so the value columns of S evolve
// independently: each wave owns NCT 16-column tiles of one (batch, head) and
// keeps its part of S, U and O in matrix-core accumulators. The accumulator
// layout is the right-operand layout of the next product (gdn2_frag.h), so
// the chain never stages S or U through LDS and needs no barrier between
// waves; the only shared data are the record's left operands, copied once per
// chunk from the workspace into LDS by direct-to-LDS loads, double-buffered so
// that chunk n+1 is in flight while chunk n is computed.

#include "gdn2_frag.h"
#include "gdn2_internal.h"

namespace gdn2 {

template <int DK, int C, bool F32IN, int NCT, int NWV>
struct ChainCfg {
  using Rec = Record<DK, C, F32IN, 0>;
  using F = Frag<F32IN>;
  static constexpr int kThreads = NWV * kWave;
  static constexpr int RC = C / 16, RK = DK / 16;
  static constexpr int NBUF = 2 * Rec::kBytes <= 160 * 1024 ? 2 : 1;
  static constexpr int kLdsBytes = NBUF * Rec::kBytes;
  static constexpr bool kFits = kLdsBytes <= 160 * 1024;
  static constexpr int kCols = 16 * NCT * NWV;  // value columns per workgroup
};

// Copy `units` 1 KB units from global src to LDS dst, units dealt round-robin
// to the nw waves (direct-to-LDS loads; the caller waits on vmcnt).
__device__ __forceinline__ void dma_units(const char* src, char* dst, int units, int wid, int nw) {
  const int l = lane_id();
  for (int t = wid; t < units; t += nw) {
    __builtin_amdgcn_global_load_lds(src + (int64_t)t * 1024 + 16 * l,
                                     (__attribute__((address_space(3))) void*)(dst + t * 1024), 16, 0, 0);
  }
}

// all vector-memory operations of this wave have completed (gfx9 encoding:
// vmcnt = 0, expcnt and lgkmcnt unconstrained)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DK, int C, bool F32IN, int NCT, int NWV>
__global__ __launch_bounds__(NWV * 64) void gdn2_chain_fwd_kernel(FwdArgs a, const char* rec_base,
                                                                 const float* ut_base) {
  using Cfg = ChainCfg<DK, C, F32IN, NCT, NWV>;
  using Rec = typename Cfg::Rec;
  using F = Frag<F32IN>;
  constexpr int RC = Cfg::RC, RK = Cfg::RK, UK = Rec::UK, UC = Rec::UC;
  constexpr int KU = F::KU;

  __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;

  // block -> (batch*head, column group); the column groups of one head share an XCD
  const int Dv = a.Dv, T = a.T, H = a.H;
  const int ncg = Dv / Cfg::kCols;
  const int nbh = a.B * H;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int bh = (slot / ncg) * 8 + xcd, cg = slot % ncg;
  if (bh >= nbh) return;
  const int bi = bh / H, h = bh - bi * H;
  const int NC = (T + C - 1) / C;
  const int j0 = cg * Cfg::kCols + wid * 16 * NCT;  // first column of this wave
  const int64_t rowV = (int64_t)H * Dv;
  const int64_t baseV = ((int64_t)bi * T * H + h) * Dv + j0;
  const int64_t stBase = (int64_t)bh * DK * Dv + j0;
  const char* recs = rec_base + (int64_t)bh * NC * Rec::kBytes;
  const float* uts = ut_base + (int64_t)bh * NC * C * Dv;
  const int nvt = Dv / 16, jb0 = j0 / 16;

  // state tiles: rows 16*RKt + 4*lg + i, column j0 + 16*c + lr
  f32x4 accS[RK][NCT];
#pragma unroll
  for (int R = 0; R < RK; ++R)
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      accS[R][c] = zero4();
      if (a.S0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[R][c][i] = a.S0[stBase + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr];
      }
    }

  auto load_ut = [&](int nn, f32x4 (&dst)[RC][NCT]) {
    const float* u = uts + (int64_t)nn * C * Dv;
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(u + (int64_t)(R * nvt + jb0 + c) * 256 + 4 * l);
        dst[R][c] = f32x4{v.x, v.y, v.z, v.w};
      }
  };

  f32x4 utn[RC][NCT];
  dma_units(recs, smem, Rec::kUnits, wid, NWV);
  load_ut(0, utn);

  for (int n = 0; n < NC; ++n) {
    const int t0 = n * C, Lr = min(C, T - t0);
    char* buf = smem + (Cfg::NBUF == 2 ? (n & 1) * Rec::kBytes : 0);
    wait_vm_all();
    __syncthreads();  // record n is in LDS; every wave is done with chunk n-1
    if (Cfg::NBUF == 2 && n + 1 < NC)
      dma_units(recs + (int64_t)(n + 1) * Rec::kBytes, smem + ((n + 1) & 1) * Rec::kBytes, Rec::kUnits, wid, NWV);

    if (a.chunk_states) {
      float* cs = a.chunk_states + ((int64_t)bh * NC + n) * DK * Dv + j0;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[(int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = accS[R][c][i];
    }

    f32x4 accU[RC][NCT], accO[RC][NCT];
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        accU[R][c] = utn[R][c];
        accO[R][c] = zero4();
      }
    if (n + 1 < NC) load_ut(n + 1, utn);

    const uint4* uW = reinterpret_cast<const uint4*>(buf + Rec::u0 * 1024) + l;
    const uint4* uQ = reinterpret_cast<const uint4*>(buf + Rec::u1 * 1024) + l;
    const uint4* uKb = reinterpret_cast<const uint4*>(buf + Rec::u2 * 1024) + l;
    const uint4* uP = reinterpret_cast<const uint4*>(buf + Rec::u3 * 1024) + l;
    const float* gam = reinterpret_cast<const float*>(buf + Rec::uG * 1024);

    // ---- U = Ut - W S ; O = Qs S  (contraction over Dk) ----
    if constexpr (F32IN) {
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const uint4 aw = uW[(R * UK + u) * 64], aq = uQ[(R * UK + u) * 64];
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            unit_mma(accU[R][c], aw, accS[u][c]);
            unit_mma(accO[R][c], aq, accS[u][c]);
          }
        }
    } else {
      f16x8 sb[UK][NCT];
#pragma unroll
      for (int u = 0; u < UK; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) sb[u][c] = rhs_from_acc(accS[2 * u][c], 2 * u + 1 < RK ? accS[2 * u + 1][c] : zero4());
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const uint4 aw = uW[(R * UK + u) * 64], aq = uQ[(R * UK + u) * 64];
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            unit_mma(accU[R][c], aw, sb[u][c]);
            unit_mma(accO[R][c], aq, sb[u][c]);
          }
        }
    }

    // ---- O += P U (P lower triangular: row tile R needs contraction < 16(R+1)) ;
    //      S <- Diag(gamma) S + Kb^T U  (contraction over the chunk) ----
    float gm[RK][4];
#pragma unroll
    for (int R = 0; R < RK; ++R) {
      const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * R + 4 * lg);
      gm[R][0] = g4.x; gm[R][1] = g4.y; gm[R][2] = g4.z; gm[R][3] = g4.w;
    }
    if constexpr (F32IN) {
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int u = 0; u < UC; ++u) {
          if (KU * u < 16 * (R + 1)) {
            const uint4 ap = uP[(R * UC + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accO[R][c], ap, accU[u][c]);
          }
        }
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) accS[R][c][i] *= gm[R][i];
#pragma unroll
          for (int u = 0; u < UC; ++u) unit_mma(accS[R][c], uKb[(R * UC + u) * 64], accU[u][c]);
        }
    } else {
      f16x8 ub[UC][NCT];
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) ub[u][c] = rhs_from_acc(accU[2 * u][c], 2 * u + 1 < RC ? accU[2 * u + 1][c] : zero4());
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int u = 0; u < UC; ++u) {
          if (KU * u < 16 * (R + 1)) {
            const uint4 ap = uP[(R * UC + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accO[R][c], ap, ub[u][c]);
          }
        }
#pragma unroll
      for (int R = 0; R < RK; ++R) {
        uint4 ak[UC];
#pragma unroll
        for (int u = 0; u < UC; ++u) ak[u] = uKb[(R * UC + u) * 64];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) accS[R][c][i] *= gm[R][i];
#pragma unroll
          for (int u = 0; u < UC; ++u) unit_mma(accS[R][c], ak[u], ub[u][c]);
        }
      }
    }

    // ---- o (not written when the caller only wants states) ----
#pragma unroll
    for (int R = 0; R < RC && a.o; ++R)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * R + 4 * lg + i;
        if (r < Lr) {
          float* op = a.o + baseV + (int64_t)(t0 + r) * rowV + lr;
#pragma unroll
          for (int c = 0; c < NCT; ++c) op[16 * c] = accO[R][c][i];
        }
      }

    if (Cfg::NBUF == 1 && n + 1 < NC) {
      __syncthreads();  // every wave is done reading the single buffer
      dma_units(recs + (int64_t)(n + 1) * Rec::kBytes, smem, Rec::kUnits, wid, NWV);
    }
  }

  if (a.S_final) {
#pragma unroll
    for (int R = 0; R < RK; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.S_final[stBase + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = accS[R][c][i];
  }
}

// ---------------------------------------------------------------------------
// Reverse chain of the backward: the gradient of every chunk's exit state.
//
// For L = <dO, o> + <dS_final, S_T>, the chunk relations above give, walking
// the chunks from last to first with dS the gradient of the chunk's exit state
// (the chunkwise form of the gate-aware backward, aiexpert.news method
// paragraph; arXiv 2605.22791 abstract):
//   dU = P^T dO + Kb dS,
//   dS <- Diag(gamma) dS + Qs^T dO - W^T dU      (gradient of the entry state).
// The backward record holds P^T, Kb, Qs^T, -W^T and gamma as left-operand
// units; dS and dU stay in accumulators as in the forward chain, and dO is
// gathered straight into right-operand fragments, one chunk ahead.
// dS_chunks[n] receives the exit-state gradient of chunk n; dS0 the final one.
// ---------------------------------------------------------------------------
template <int DK, int C, bool F32IN, int NCT, int NWV>
__global__ __launch_bounds__(NWV * 64) void gdn2_chain_bwd_kernel(BwdArgs a, const char* rec_base) {
  using Rec = Record<DK, C, F32IN, 1>;
  using F = Frag<F32IN>;
  constexpr int RC = C / 16, RK = DK / 16, UK = Rec::UK, UC = Rec::UC;
  constexpr int KU = F::KU;
  constexpr int kBuf = Rec::kChainBytes;  // the chain's prefix of each record
  constexpr int NBUF = 2 * kBuf <= 160 * 1024 ? 2 : 1;
  constexpr int kCols = 16 * NCT * NWV;

  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kBuf];

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int Dv = a.Dv, T = a.T, H = a.H;
  const int ncg = Dv / kCols;
  const int nbh = a.B * H;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int bh = (slot / ncg) * 8 + xcd, cg = slot % ncg;
  if (bh >= nbh) return;
  const int bi = bh / H, h = bh - bi * H;
  const int NC = (T + C - 1) / C;
  const int j0 = cg * kCols + wid * 16 * NCT;
  const int64_t rowV = (int64_t)H * Dv;
  const int64_t baseV = ((int64_t)bi * T * H + h) * Dv + j0;
  const int64_t stBase = (int64_t)bh * DK * Dv + j0;
  const char* recs = rec_base + (int64_t)bh * NC * Rec::kBytes;

  f32x4 accD[RK][NCT];
#pragma unroll
  for (int R = 0; R < RK; ++R)
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      accD[R][c] = zero4();
      if (a.dS_final) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          accD[R][c][i] = a.dS_final[stBase + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr];
      }
    }

  // dO of chunk nn as right-operand fragments (contraction over the chunk's tokens)
  constexpr int NDU = F32IN ? RC : UC;    // fragments per column tile
  constexpr int NDE = F32IN ? 4 : 8;      // elements per fragment
  using RawT = typename std::conditional<F32IN, float, uint16_t>::type;
  RawT rdo[NDU][NCT][NDE];
  auto load_do = [&](int nn) {
    const int tn = nn * C, Ln = min(C, T - tn);
#pragma unroll
    for (int u = 0; u < NDU; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int j = 0; j < NDE; ++j) {
          const int t = F32IN ? 16 * u + 4 * lg + j : KU * u + F::kslot(lg, j);
          const int64_t idx = baseV + (int64_t)(tn + t) * rowV + 16 * c + lr;
          const int64_t safe = baseV + (int64_t)tn * rowV + 16 * c + lr;  // the chunk's first row
          rdo[u][c][j] = ld_sel(static_cast<const RawT*>(a.dO), idx, safe, t < Ln);
        }
  };

  dma_units(recs + (int64_t)(NC - 1) * Rec::kBytes, smem + (NBUF == 2 ? ((NC - 1) & 1) * kBuf : 0),
            Rec::kChainUnits, wid, NWV);
  load_do(NC - 1);

  for (int n = NC - 1; n >= 0; --n) {
    char* buf = smem + (NBUF == 2 ? (n & 1) * kBuf : 0);
    wait_vm_all();
    __syncthreads();  // record n is in LDS; every wave is done with chunk n+1
    if (NBUF == 2 && n > 0)
      dma_units(recs + (int64_t)(n - 1) * Rec::kBytes, smem + ((n - 1) & 1) * kBuf, Rec::kChainUnits, wid, NWV);

    {
      float* ws = a.dS_chunks + ((int64_t)bh * NC + n) * DK * Dv + j0;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) ws[(int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = accD[R][c][i];
    }

    // this chunk's dO fragments; the previous chunk's start loading
    using DoF = typename std::conditional<F32IN, f32x4, f16x8>::type;
    DoF dof[NDU][NCT];
#pragma unroll
    for (int u = 0; u < NDU; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int j = 0; j < NDE; ++j) {
          if constexpr (F32IN) dof[u][c][j] = rdo[u][c][j];
          else dof[u][c][j] = static_cast<_Float16>(bf16_bits_to_f32(rdo[u][c][j]));
        }
    if (n > 0) load_do(n - 1);

    const uint4* uPT = reinterpret_cast<const uint4*>(buf + Rec::u0 * 1024) + l;
    const uint4* uKb = reinterpret_cast<const uint4*>(buf + Rec::u1 * 1024) + l;
    const uint4* uQT = reinterpret_cast<const uint4*>(buf + Rec::u2 * 1024) + l;
    const uint4* uWT = reinterpret_cast<const uint4*>(buf + Rec::u3 * 1024) + l;
    const float* gam = reinterpret_cast<const float*>(buf + Rec::uG * 1024);

    // ---- dU = P^T dO + Kb dS  (P^T row tile R is zero below contraction 16R) ----
    f32x4 accU[RC][NCT];
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c) accU[R][c] = zero4();
    if constexpr (F32IN) {
#pragma unroll
      for (int R = 0; R < RC; ++R) {
#pragma unroll
        for (int u = 0; u < UC; ++u) {
          if (KU * u + KU - 1 >= 16 * R) {
            const uint4 ap = uPT[(R * UC + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], ap, dof[u][c]);
          }
        }
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const uint4 ak = uKb[(R * UK + u) * 64];
#pragma unroll
          for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], ak, accD[u][c]);
        }
      }
    } else {
      f16x8 sb[UK][NCT];
#pragma unroll
      for (int u = 0; u < UK; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) sb[u][c] = rhs_from_acc(accD[2 * u][c], 2 * u + 1 < RK ? accD[2 * u + 1][c] : zero4());
#pragma unroll
      for (int R = 0; R < RC; ++R) {
#pragma unroll
        for (int u = 0; u < UC; ++u) {
          if (KU * u + KU - 1 >= 16 * R) {
            const uint4 ap = uPT[(R * UC + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], ap, dof[u][c]);
          }
        }
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const uint4 ak = uKb[(R * UK + u) * 64];
#pragma unroll
          for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], ak, sb[u][c]);
        }
      }
    }

    // ---- dS <- Diag(gamma) dS + Qs^T dO - W^T dU ----
    float gm[RK][4];
#pragma unroll
    for (int R = 0; R < RK; ++R) {
      const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * R + 4 * lg);
      gm[R][0] = g4.x; gm[R][1] = g4.y; gm[R][2] = g4.z; gm[R][3] = g4.w;
    }
    if constexpr (F32IN) {
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) accD[R][c][i] *= gm[R][i];
#pragma unroll
          for (int u = 0; u < UC; ++u) {
            unit_mma(accD[R][c], uQT[(R * UC + u) * 64], dof[u][c]);
            unit_mma(accD[R][c], uWT[(R * UC + u) * 64], accU[u][c]);
          }
        }
    } else {
      f16x8 ub[UC][NCT];
#pragma unroll
      for (int u = 0; u < UC; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) ub[u][c] = rhs_from_acc(accU[2 * u][c], 2 * u + 1 < RC ? accU[2 * u + 1][c] : zero4());
#pragma unroll
      for (int R = 0; R < RK; ++R) {
        uint4 aq[UC], aw[UC];
#pragma unroll
        for (int u = 0; u < UC; ++u) {
          aq[u] = uQT[(R * UC + u) * 64];
          aw[u] = uWT[(R * UC + u) * 64];
        }
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) accD[R][c][i] *= gm[R][i];
#pragma unroll
          for (int u = 0; u < UC; ++u) {
            unit_mma(accD[R][c], aq[u], dof[u][c]);
            unit_mma(accD[R][c], aw[u], ub[u][c]);
          }
        }
      }
    }

    if (NBUF == 1 && n > 0) {
      __syncthreads();  // every wave is done reading the single buffer
      dma_units(recs + (int64_t)(n - 1) * Rec::kBytes, smem, Rec::kChainUnits, wid, NWV);
    }
  }

  if (a.dS0) {
#pragma unroll
    for (int R = 0; R < RK; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dS0[stBase + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = accD[R][c][i];
  }
}

// ---------------------------------------------------------------------------
// dispatch: NCT = 2 (32 columns per wave) when Dv allows, NWV waves so that
// the grid has at least ~256 workgroups when it can
// ---------------------------------------------------------------------------
template <int DK, int C, bool F32IN, int NCT, int NWV>
static hipError_t launch_chain_t(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  using Cfg = ChainCfg<DK, C, F32IN, NCT, NWV>;
  if constexpr (!Cfg::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int ncg = a.Dv / Cfg::kCols;
    const int nbh = a.B * a.H;
    const int grid = ((nbh + 7) / 8) * 8 * ncg;
    hipLaunchKernelGGL((gdn2_chain_fwd_kernel<DK, C, F32IN, NCT, NWV>), dim3(grid), dim3(Cfg::kThreads), 0, s, a,
                       rec, ut);
    return hipGetLastError();
  }
}

template <int DK, int C, bool F32IN>
static hipError_t launch_chain_c(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  const int nbh = a.B * a.H;
  if (a.Dv == 16) return launch_chain_t<DK, C, F32IN, 1, 1>(a, rec, ut, s);
  // 32 columns per wave; as many waves per workgroup as keep >= 256 workgroups
  const int tiles = a.Dv / 32;  // wave tiles per head
  if (tiles >= 2 && nbh * (tiles / 2) >= 256) return launch_chain_t<DK, C, F32IN, 2, 2>(a, rec, ut, s);
  if (nbh * tiles >= 256) return launch_chain_t<DK, C, F32IN, 2, 1>(a, rec, ut, s);
  return launch_chain_t<DK, C, F32IN, 1, 1>(a, rec, ut, s);  // few heads: 16 columns per workgroup
}

template <int DK, bool F32IN>
static hipError_t launch_chain_k(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_chain_c<DK, 16, F32IN>(a, rec, ut, s);
    case 32: return launch_chain_c<DK, 32, F32IN>(a, rec, ut, s);
    case 64: return launch_chain_c<DK, 64, F32IN>(a, rec, ut, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_chain_f(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_chain_k<16, F32IN>(a, rec, ut, s);
    case 32: return launch_chain_k<32, F32IN>(a, rec, ut, s);
    case 64: return launch_chain_k<64, F32IN>(a, rec, ut, s);
    case 128: return launch_chain_k<128, F32IN>(a, rec, ut, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chain_fwd(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  return a.f32_inputs ? launch_chain_f<true>(a, rec, ut, s) : launch_chain_f<false>(a, rec, ut, s);
}

template <int DK, int C, bool F32IN, int NCT, int NWV>
static hipError_t launch_chain_bwd_t(const BwdArgs& a, const char* rec, hipStream_t s) {
  using Rec = Record<DK, C, F32IN, 1>;
  if constexpr (Rec::kChainBytes > 160 * 1024) {
    return hipErrorInvalidConfiguration;
  } else {
    const int ncg = a.Dv / (16 * NCT * NWV);
    const int nbh = a.B * a.H;
    const int grid = ((nbh + 7) / 8) * 8 * ncg;
    hipLaunchKernelGGL((gdn2_chain_bwd_kernel<DK, C, F32IN, NCT, NWV>), dim3(grid), dim3(NWV * 64), 0, s, a, rec);
    return hipGetLastError();
  }
}

template <int DK, int C, bool F32IN>
static hipError_t launch_chain_bwd_c(const BwdArgs& a, const char* rec, hipStream_t s) {
  const int nbh = a.B * a.H;
  if (a.Dv == 16) return launch_chain_bwd_t<DK, C, F32IN, 1, 1>(a, rec, s);
  const int tiles = a.Dv / 32;
  if (tiles >= 2 && nbh * (tiles / 2) >= 256) return launch_chain_bwd_t<DK, C, F32IN, 2, 2>(a, rec, s);
  if (nbh * tiles >= 256) return launch_chain_bwd_t<DK, C, F32IN, 2, 1>(a, rec, s);
  return launch_chain_bwd_t<DK, C, F32IN, 1, 1>(a, rec, s);
}

template <int DK, bool F32IN>
static hipError_t launch_chain_bwd_k(const BwdArgs& a, const char* rec, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_chain_bwd_c<DK, 16, F32IN>(a, rec, s);
    case 32: return launch_chain_bwd_c<DK, 32, F32IN>(a, rec, s);
    case 64: return launch_chain_bwd_c<DK, 64, F32IN>(a, rec, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_chain_bwd_f(const BwdArgs& a, const char* rec, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_chain_bwd_k<16, F32IN>(a, rec, s);
    case 32: return launch_chain_bwd_k<32, F32IN>(a, rec, s);
    case 64: return launch_chain_bwd_k<64, F32IN>(a, rec, s);
    case 128: return launch_chain_bwd_k<128, F32IN>(a, rec, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chain_bwd(const BwdArgs& a, const char* rec, hipStream_t s) {
  return a.f32_inputs ? launch_chain_bwd_f<true>(a, rec, s) : launch_chain_bwd_f<false>(a, rec, s);
}

}  // namespace gdn2
