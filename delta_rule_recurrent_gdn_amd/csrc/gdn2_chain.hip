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
//
// Segmented (two-level) form, for few (batch, head) pairs and long sequences:
// the chunk map is affine in the entry state, S_out = M S_in + N with
// M = prod (Diag(gamma) - Kb^T W) and N the exit state from a zero entry. A
// head's chunks are cut into segments of L chunks; (1) every segment runs the
// chain from a zero state on its value columns (-> N) and on DK identity
// columns with no input (-> M), all segments in parallel; (2) a short
// sequential pass composes S_in(s+1) = M_s S_in(s) + N_s in fp32; (3) every
// segment runs again from its true entry state and writes o, the chunk entry
// states and the final state. Same arithmetic per chunk; the sequential depth
// drops from NC chunks to about 2L + NC/L.

#include <type_traits>

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

// The same, over units [0, units) less the ranges [s0, e0) and [s1, e1) (wave-uniform bounds).
__device__ __forceinline__ void dma_units_skip(const char* src, char* dst, int units, int s0, int e0, int s1, int e1,
                                               int wid, int nw) {
  const int l = lane_id();
  for (int t = wid; t < units; t += nw) {
    if ((t >= s0 && t < e0) || (t >= s1 && t < e1)) continue;
    __builtin_amdgcn_global_load_lds(src + (int64_t)t * 1024 + 16 * l,
                                     (__attribute__((address_space(3))) void*)(dst + t * 1024), 16, 0, 0);
  }
}

// Helper waves of the plain reverse chain (one workgroup per CU): they take the
// record copies off the column waves, which also gather dO (1.41 -> 1.38 ms for
// the B8 H16 T4096 backward; four helpers: 1.39 ms). The forward chain has none:
// its four column waves need more than the 256 registers a wave may hold when a
// SIMD runs two, and with two column waves helpers made it slower.
constexpr int kChainHelpers = 2;

// all vector-memory operations of this wave have completed (gfx9 encoding:
// vmcnt = 0, expcnt and lgkmcnt unconstrained)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Two-level chain: waves (of 16 value columns) per workgroup of the map and run passes. With four the
// passes need twice the workgroups at one per CU, and the map pass a second round (B1 H16 T64K forward
// 1.74 -> 1.85 ms).
constexpr int kSegWaves = 8;

// threads of the segment composition: eight waves, each one 16-row tile of the state's 32 columns
// (its products are a chain of dependent fp32 matrix-core steps; two waves per SIMD overlap theirs)
constexpr int kComposeThreads = 512;

// Segment slot and column group of a workgroup of the two-level chain's passes. The column groups of one
// segment take workgroups 8 apart, so that they run on one XCD and read each record through its L2 once
// (B1 H16 T64K forward 1.77 -> 1.74 ms); -1 past the last slot (the grid is rounded up to whole groups of
// 8). Slots: dense, (batch*head, s) with s < nseg (map pass: nseg - 1); packed, (head, global segment).
__device__ __forceinline__ int seg_block_item(const Varlen& vl, const SegArgs& sg, int nbh, int H, int ncg,
                                              int& cg) {
  const int nitems = vl.cu == nullptr ? nbh * (sg.mode == kSegMap ? sg.nseg - 1 : sg.nseg) : H * vl.max_segs;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int item = (slot / ncg) * 8 + xcd;
  cg = slot - (slot / ncg) * ncg;
  return item < nitems ? item : -1;
}
// Workgroups of a two-level pass over `items` slots of ncg column groups each.
inline unsigned seg_grid(int64_t items, int ncg) { return (unsigned)(((items + 7) / 8) * 8 * ncg); }

// NHW helper waves: waves past the NWV column waves own no columns and only
// copy the next record into LDS (used by the plain reverse chain; see
// kChainHelpers).
// MAP: the segmented map pass (sg.mode == kSegMap), compiled on its own: it writes no o.
template <int DK, int C, bool F32IN, int NCT, int NWV, bool SEG, int NHW = 0, bool MAP = false>
__global__ __launch_bounds__((NWV + NHW) * 64) void gdn2_chain_fwd_kernel(FwdArgs a, const char* rec_base,
                                                                          const float* ut_base, SegArgs sg) {
  static_assert(!MAP || (SEG && NHW == 0), "the map pass is a segmented pass without helper waves");
  using Cfg = ChainCfg<DK, C, F32IN, NCT, NWV>;
  using Rec = typename Cfg::Rec;
  using F = Frag<F32IN>;
  constexpr int RC = Cfg::RC, RK = Cfg::RK, UK = Rec::UK, UC = Rec::UC;
  constexpr int KU = F::KU;

  // two record buffers (one when two do not fit), as separate arrays: see the step loop
  __shared__ __attribute__((aligned(1024))) char smemA[Rec::kBytes];
  __shared__ __attribute__((aligned(1024))) char smemB[Cfg::NBUF == 2 ? Rec::kBytes : 16];
  char* const smem = smemA;

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;

  const int Dv = a.Dv, T = a.T, H = a.H;
  const int nbh = seq_items(a.vl, a.B, H);
  const int NC = (T + C - 1) / C;
  int bh, cg, n_begin = 0, n_end = NC;
  int64_t segIdx = 0;               // this segment's slot in M, N, S_in
  bool seg_first = true, seg_last = true;
  if constexpr (SEG) {
    // block -> (segment, column group); the columns are the value columns,
    // followed in the map pass by DK identity columns. Dense: segments
    // (batch*head, s), s < nseg (map pass: s < nseg - 1); packed sequences:
    // (head, global segment), a sequence's last segment skipped by the map pass.
    const int ncg = ((sg.mode == kSegMap ? Dv + DK : Dv) + Cfg::kCols - 1) / Cfg::kCols;
    const int item = seg_block_item(a.vl, sg, nbh, H, ncg, cg);
    if (item < 0) return;
    int local;
    if (a.vl.cu == nullptr) {
      const int nsb = sg.mode == kSegMap ? sg.nseg - 1 : sg.nseg;
      bh = item / nsb;
      local = item - bh * nsb;
      segIdx = (int64_t)bh * sg.nseg + local;
      seg_last = local == sg.nseg - 1;
    } else {
      const int h = item / a.vl.max_segs, gsg = item - h * a.vl.max_segs;
      const int sq = a.vl.seg_seq[gsg];
      if (sq < 0) return;  // past the last segment
      local = gsg - a.vl.seg_first[sq];
      seg_last = gsg == a.vl.seg_first[sq + 1] - 1;
      if (sg.mode == kSegMap && seg_last) return;  // no map needed after a sequence's last segment
      bh = sq * H + h;
      segIdx = (int64_t)h * a.vl.max_segs + gsg;
    }
    seg_first = local == 0;
    n_begin = local * sg.seg_len;
    n_end = n_begin + sg.seg_len;  // clipped to the sequence below
  } else {
    // block -> (batch*head, column group); the column groups of one head share an XCD
    const int ncg = Dv / Cfg::kCols;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bh = (slot / ncg) * 8 + xcd;
    cg = slot % ncg;
    if (bh >= nbh) return;
  }
  // the (batch row or packed sequence, head) walked here: its chunks, tokens and states
  const SeqLoc sl = seq_loc(a.vl, T, H, DK, Dv, C, bh);
  n_end = SEG ? min(n_end, sl.nchunks) : sl.nchunks;
  const int j0 = cg * Cfg::kCols + wid * 16 * NCT;  // first column of this wave
  // segmented: waves past the columns only copy records; identity columns (j0 >= Dv, map pass) have no input;
  // plain: the helper waves only copy records
  const bool active = SEG ? j0 < (sg.mode == kSegMap ? Dv + DK : Dv) : wid < NWV;
  const bool ident = SEG && j0 >= Dv;
  const int64_t rowV = (int64_t)H * Dv;
  const int64_t baseV = sl.baseV + j0;
  const int64_t stBase = sl.state * DK * Dv + j0;
  const char* recs = rec_base + sl.item0 * Rec::kBytes;
  // T (w v): fp32 tiles for fp32 inputs, fp16 for 16-bit ones, held packed until their step uses them
  using UtReg = typename std::conditional<F32IN, f32x4, uint2>::type;
  const char* uts = reinterpret_cast<const char*>(ut_base) + sl.item0 * C * Dv * (F32IN ? 4 : 2);
  const int nvt = Dv / 16, jb0 = j0 / 16;

  // state tiles: rows 16*RKt + 4*lg + i, column j0 + 16*c + lr
  // entry: S0 (or zero); segmented map pass: zero, identity on the identity
  // columns; segmented run: S0 for the first segment, else the composed entry
  const float* Sent = a.S0;
  int64_t sOff = stBase;
  if constexpr (SEG) {
    if (sg.mode == kSegMap) {
      Sent = nullptr;
    } else if (!seg_first) {
      Sent = sg.S_in;
      sOff = segIdx * DK * Dv + j0;
    }
  }
  f32x4 accS[RK][NCT];
#pragma unroll
  for (int R = 0; R < RK; ++R)
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      accS[R][c] = zero4();
      if (ident) {
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[R][c][i] = (16 * R + 4 * lg + i == j0 - Dv + 16 * c + lr) ? 1.f : 0.f;
      } else if (Sent && active) {
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[R][c][i] = Sent[sOff + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr];
      }
    }

  auto load_ut = [&](int nn, UtReg (&dst)[RC][NCT]) {
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int64_t e = (int64_t)nn * C * Dv + (int64_t)(R * nvt + jb0 + c) * 256 + 4 * l;
        if constexpr (F32IN) {
          const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(uts) + e);
          dst[R][c] = f32x4{v.x, v.y, v.z, v.w};
        } else {
          dst[R][c] = *reinterpret_cast<const uint2*>(reinterpret_cast<const _Float16*>(uts) + e);
        }
      }
  };

  // the value columns' outputs: every pass but the segmented map pass
  const bool outs = SEG ? (sg.mode == kSegRun && active) : active;
  const bool has_ut = active && !ident;
  // record copies: by the helper waves when there are any, else by all waves. The segmented map pass
  // (MAP) computes no o: it needs neither the decayed q nor the causal term, so it copies neither into
  // LDS and skips their products (24 of the 57 units of a bf16 d = 128 record, a third of the products)
  auto dma = [&](const char* src, char* dst) {
    if constexpr (MAP) {
      dma_units_skip(src, dst, Rec::kUnits, Rec::u1, Rec::u2, Rec::u3, Rec::uG, wid, NWV);
    } else if constexpr (NHW > 0) {
      if (wid >= NWV) dma_units(src, dst, Rec::kUnits, wid - NWV, NHW);
    } else {
      dma_units(src, dst, Rec::kUnits, wid, NWV);
    }
  };
  UtReg utA[RC][NCT], utB[RC][NCT];
  auto ut_f32 = [](const UtReg& x) -> f32x4 {
    if constexpr (F32IN) {
      return x;
    } else {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 h = __builtin_bit_cast(h4, x);
      return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                   static_cast<float>(h[3])};
    }
  };
  if (n_begin < n_end) {  // an empty packed sequence has no chunk: S_final = S0
    dma(recs + (int64_t)n_begin * Rec::kBytes, smem);
    if (has_ut) load_ut(n_begin, utA);
  }

  // o of chunk n is stored at the start of step n + 1: every step begins by
  // waiting for all of the wave's vector-memory operations (the next record and
  // T (w v) loads), and stores count among them, so stores issued at the end of
  // a step would put their full write latency on the chain. (Not in the
  // segmented kernel, whose 8-wave workgroups have no registers to spare.)
  constexpr bool kDefer = !SEG;
  f32x4 oPrev[RC][NCT];
  int t0Prev = 0, LrPrev = 0;
  bool oPend = false;
  auto store_o = [&]() {
#pragma unroll
    for (int R = 0; R < RC; ++R)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * R + 4 * lg + i;
        if (r < LrPrev) {
          float* op = a.o + baseV + (int64_t)(t0Prev + r) * rowV + lr;
#pragma unroll
          for (int c = 0; c < NCT; ++c) op[16 * c] = oPrev[R][c][i];
        }
      }
  };

  // one chain step: record n in buf, the next record's copy into nbuf; T (w v) of chunk n in utc, the next
  // chunk's loaded into utx
  auto step = [&](const int n, char* buf, char* nbuf, UtReg (&utc)[RC][NCT], UtReg (&utx)[RC][NCT])
                  __attribute__((always_inline)) {
    const int t0 = sl.tok0 + n * C, Lr = min(C, sl.len - n * C);
    wait_vm_all();
    __syncthreads();  // record n is in LDS; every wave is done with chunk n-1
    if (Cfg::NBUF == 2 && n + 1 < n_end)
      dma(recs + (int64_t)(n + 1) * Rec::kBytes, nbuf);
    if (oPend) store_o();

    if (a.states16 && outs) {
      _Float16* cs = a.states16 + (sl.item0 + n) * DK * Dv + j0;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            cs[(int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = static_cast<_Float16>(accS[R][c][i]);
    } else if (a.chunk_states && outs) {
      float* cs = a.chunk_states + (sl.item0 + n) * DK * Dv + j0;
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
        accU[R][c] = has_ut ? ut_f32(utc[R][c]) : zero4();
        accO[R][c] = zero4();
      }
    if (has_ut && n + 1 < n_end) load_ut(n + 1, utx);
    if (active) {

    const uint4* uW = reinterpret_cast<const uint4*>(buf + Rec::u0 * 1024) + l;
    const uint4* uQ = reinterpret_cast<const uint4*>(buf + Rec::u1 * 1024) + l;
    const uint4* uKb = reinterpret_cast<const uint4*>(buf + Rec::u2 * 1024) + l;
    const uint4* uP = reinterpret_cast<const uint4*>(buf + Rec::u3 * 1024) + l;
    const float* gam = reinterpret_cast<const float*>(buf + Rec::uG * 1024);

    // ---- U = Ut - W S ; O = Qs S  (contraction over Dk) ----
    if constexpr (!MAP) {
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
          for (int c = 0; c < NCT; ++c)
            sb[u][c] = rhs_from_acc(accS[2 * u][c], 2 * u + 1 < RK ? accS[2 * u + 1][c] : zero4());
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
    } else {  // map pass: U only
      if constexpr (F32IN) {
#pragma unroll
        for (int R = 0; R < RC; ++R)
#pragma unroll
          for (int u = 0; u < UK; ++u) {
            const uint4 aw = uW[(R * UK + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], aw, accS[u][c]);
          }
      } else {
        f16x8 sb[UK][NCT];
#pragma unroll
        for (int u = 0; u < UK; ++u)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            sb[u][c] = rhs_from_acc(accS[2 * u][c], 2 * u + 1 < RK ? accS[2 * u + 1][c] : zero4());
#pragma unroll
        for (int R = 0; R < RC; ++R)
#pragma unroll
          for (int u = 0; u < UK; ++u) {
            const uint4 aw = uW[(R * UK + u) * 64];
#pragma unroll
            for (int c = 0; c < NCT; ++c) unit_mma(accU[R][c], aw, sb[u][c]);
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
      if constexpr (!MAP) {
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
      if constexpr (!MAP) {
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

    // ---- o (not written when the caller only wants states): stored next step ----
    if (a.o && outs) {
#pragma unroll
      for (int R = 0; R < RC; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c) oPrev[R][c] = accO[R][c];
      t0Prev = t0;
      LrPrev = Lr;
      oPend = true;
      if constexpr (!kDefer) {
        store_o();
        oPend = false;
      }
    }
    }  // active

    if (Cfg::NBUF == 1 && n + 1 < n_end) {
      __syncthreads();  // every wave is done reading the single buffer
      dma(recs + (int64_t)(n + 1) * Rec::kBytes, smem);
    }
  };
  // Steps in pairs, so that every record copy and every LDS read names its buffer, and every T (w v) load
  // its registers, statically. With the buffer chosen at run time the compiler waited, before the first
  // LDS read of each step, for every vector-memory operation then in flight (the next record's copy
  // included), and moving the loaded T (w v) into the registers of the next step forced the same wait.
  char* const nextA = Cfg::NBUF == 2 ? smemB : smemA;
  for (int n = n_begin; n < n_end; n += 2) {
    step(n, smemA, nextA, utA, utB);
    if (n + 1 < n_end) step(n + 1, nextA, smemA, utB, utA);
  }
  if (oPend) store_o();  // the last chunk's o

  if constexpr (SEG) {
    if (sg.mode == kSegMap && active) {
      // exit of a zero-entry segment: N (value columns) or M (identity columns)
      const int64_t sb = segIdx;
      float* dst = ident ? sg.M + sb * DK * DK + (j0 - Dv) : sg.N + sb * DK * Dv + j0;
      const int ld = ident ? DK : Dv;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * R + 4 * lg + i) * ld + 16 * c + lr] = accS[R][c][i];
      return;
    }
    if (!seg_last || !active) return;
  }
  if (!active) return;  // helper waves
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
//
// Segmented (two-level) form, the mirror image of the forward's: per chunk
// dS_entry = (Diag(gamma) - W^T Kb) dS_exit + (terms in dO), so a segment maps
// the gradient at its exit to the one at its entry, dS_in = M dS_out + N.
// (1) every segment but the first in time runs from a zero exit gradient on
// its value columns (-> N) and on DK identity columns without dO (-> M);
// (2) a short pass composes dS_out(s-1) = M_s dS_out(s) + N_s backwards from
// dS_final; (3) every segment runs again from its true exit gradient, writing
// its chunks' exit gradients and (first segment) dS0.
// ---------------------------------------------------------------------------
template <int DK, int C, bool F32IN, int NCT, int NWV, bool SEG, int NHW = 0>
__global__ __launch_bounds__((NWV + NHW) * 64) void gdn2_chain_bwd_kernel(BwdArgs a, const char* rec_base,
                                                                          SegArgs sg) {
  using Rec = Record<DK, C, F32IN, 1>;
  using F = Frag<F32IN>;
  constexpr int RC = C / 16, RK = DK / 16, UK = Rec::UK, UC = Rec::UC;
  constexpr int KU = F::KU;
  constexpr int kBuf = Rec::kChainBytes;  // the chain's prefix of each record
  constexpr int NBUF = 2 * kBuf <= 160 * 1024 ? 2 : 1;
  constexpr int kCols = 16 * NCT * NWV;

  // record buffers as separate arrays, as in the forward chain
  __shared__ __attribute__((aligned(1024))) char smemA[kBuf];
  __shared__ __attribute__((aligned(1024))) char smemB[NBUF == 2 ? kBuf : 16];
  char* const smem = smemA;

  const int tid = threadIdx.x, wid = tid / kWave, l = tid & (kWave - 1);
  const int lr = l & 15, lg = l >> 4;
  const int Dv = a.Dv, T = a.T, H = a.H;
  const int nbh = seq_items(a.vl, a.B, H);
  int bh, cg, n_begin = 0, n_end = 1 << 30;
  int64_t segIdx = 0;               // this segment's slot in M, N, S_in (here: exit gradients)
  bool seg_first = true, seg_last = true;
  if constexpr (SEG) {
    // block -> (segment, column group) as in the forward's segmented chain, except that the map
    // pass covers every segment but the FIRST of each (batch row or sequence, head)
    const int ncg = ((sg.mode == kSegMap ? Dv + DK : Dv) + kCols - 1) / kCols;
    const int item = seg_block_item(a.vl, sg, nbh, H, ncg, cg);
    if (item < 0) return;
    int local;
    if (a.vl.cu == nullptr) {
      const int nsb = sg.mode == kSegMap ? sg.nseg - 1 : sg.nseg;
      bh = item / nsb;
      local = item - bh * nsb + (sg.mode == kSegMap ? 1 : 0);
      segIdx = (int64_t)bh * sg.nseg + local;
      seg_last = local == sg.nseg - 1;
    } else {
      const int h = item / a.vl.max_segs, gsg = item - h * a.vl.max_segs;
      const int sq = a.vl.seg_seq[gsg];
      if (sq < 0) return;  // past the last segment
      local = gsg - a.vl.seg_first[sq];
      seg_last = gsg == a.vl.seg_first[sq + 1] - 1;
      if (sg.mode == kSegMap && local == 0) return;  // no map needed before a sequence's first segment
      bh = sq * H + h;
      segIdx = (int64_t)h * a.vl.max_segs + gsg;
    }
    seg_first = local == 0;
    n_begin = local * sg.seg_len;
    n_end = n_begin + sg.seg_len;
  } else {
    const int ncg = Dv / kCols;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bh = (slot / ncg) * 8 + xcd;
    cg = slot % ncg;
    if (bh >= nbh) return;
  }
  // the (batch row or packed sequence, head) walked here: its chunks, tokens and states
  const SeqLoc sl = seq_loc(a.vl, T, H, DK, Dv, C, bh);
  n_end = min(n_end, sl.nchunks);
  // 16-bit inputs: dO and dS_final enter times a power of two (grad_scale), dS0 leaves without it
  const float gsc = F32IN ? 1.f : grad_scale(a.gscale, sl.state);
  const int j0 = cg * kCols + wid * 16 * NCT;
  // segmented: waves past the columns only copy records; identity columns (map pass) have no dO;
  // plain: the helper waves (NHW, as in the forward chain) only copy records
  const bool active = SEG ? j0 < (sg.mode == kSegMap ? Dv + DK : Dv) : wid < NWV;
  const bool ident = SEG && j0 >= Dv;
  const bool outs = SEG ? (sg.mode == kSegRun && active) : active;  // exit gradients and dS0
  const bool has_do = active && !ident;
  // record copies (the chain's prefix of each record): by the helper waves when there are any
  auto dma = [&](const char* src, char* dst) {
    if constexpr (NHW > 0) {
      if (wid >= NWV) dma_units(src, dst, Rec::kChainUnits, wid - NWV, NHW);
    } else {
      dma_units(src, dst, Rec::kChainUnits, wid, NWV);
    }
  };
  const int64_t rowV = (int64_t)H * Dv;
  const int64_t baseV = sl.baseV + j0;
  const int64_t stBase = sl.state * DK * Dv + j0;
  const char* recs = rec_base + sl.item0 * Rec::kBytes;

  // carried gradient: dS_final (or zero); segmented map pass: zero, identity on the identity
  // columns; segmented run: dS_final for the last segment, else the composed exit gradient
  const float* Gent = a.dS_final;
  int64_t gOff = stBase;
  if constexpr (SEG) {
    if (sg.mode == kSegMap) {
      Gent = nullptr;
    } else if (!seg_last) {
      Gent = sg.S_in;
      gOff = segIdx * DK * Dv + j0;
    }
  }
  f32x4 accD[RK][NCT];
#pragma unroll
  for (int R = 0; R < RK; ++R)
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      accD[R][c] = zero4();
      if (ident) {
#pragma unroll
        for (int i = 0; i < 4; ++i) accD[R][c][i] = (16 * R + 4 * lg + i == j0 - Dv + 16 * c + lr) ? 1.f : 0.f;
      } else if (Gent && active) {
        const float gin = Gent == a.dS_final ? gsc : 1.f;  // a composed exit gradient is already scaled
#pragma unroll
        for (int i = 0; i < 4; ++i)
          accD[R][c][i] = gin * Gent[gOff + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr];
      }
    }

  // dO of chunk nn as right-operand fragments (contraction over the chunk's tokens): fetched one step
  // ahead as raw values (rows past the sequence read the chunk's first row) and zeroed past the sequence
  // when they are used, so that nothing waits for the loads in the step that issues them
  constexpr int NDU = F32IN ? RC : UC;    // fragments per column tile
  constexpr int NDE = F32IN ? 4 : 8;      // elements per fragment
  // (bf16 bits one per register: packed two to a register, the loads are waited for at once; the
  // segmented kernel's 8-wave workgroups keep them packed, with one dO set, for want of registers)
  using RawT = typename std::conditional<F32IN, float, typename std::conditional<SEG, uint16_t, uint32_t>::type>::type;
  auto do_row = [&](int u, int j) { return F32IN ? 16 * u + 4 * lg + j : KU * u + F::kslot(lg, j); };
  RawT rdoA[NDU][NCT][NDE], rdoB[NDU][NCT][NDE];
  auto load_do = [&](int nn, RawT (&dst)[NDU][NCT][NDE]) {
    const int tn = sl.tok0 + nn * C, Ln = min(C, sl.len - nn * C);
#pragma unroll
    for (int u = 0; u < NDU; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int j = 0; j < NDE; ++j) {
          const int t = do_row(u, j);
          const int64_t idx = baseV + (int64_t)(tn + t) * rowV + 16 * c + lr;
          const int64_t safe = baseV + (int64_t)tn * rowV + 16 * c + lr;  // the chunk's first row
          if constexpr (SEG) dst[u][c][j] = ld_sel(static_cast<const RawT*>(a.dO), idx, safe, t < Ln);
          else if constexpr (F32IN) dst[u][c][j] = static_cast<const float*>(a.dO)[t < Ln ? idx : safe];
          else dst[u][c][j] = static_cast<const uint16_t*>(a.dO)[t < Ln ? idx : safe];
        }
  };

  if (n_begin < n_end) {  // an empty packed sequence has no chunk: dS0 = dS_final
    dma(recs + (int64_t)(n_end - 1) * Rec::kBytes, smem);
    if (has_do) load_do(n_end - 1, rdoA);
  }

  // one chain step: record n in buf, the previous record's copy into nbuf; dO of chunk n in rdc, the
  // previous chunk's loaded into rdx
  auto step = [&](const int n, char* buf, char* nbuf, RawT (&rdc)[NDU][NCT][NDE], RawT (&rdx)[NDU][NCT][NDE])
                  __attribute__((always_inline)) {
    wait_vm_all();
    __syncthreads();  // record n is in LDS; every wave is done with chunk n+1
    if (NBUF == 2 && n > n_begin)
      dma(recs + (int64_t)(n - 1) * Rec::kBytes, nbuf);

    if (outs) {
      using SdT = typename std::conditional<F32IN, float, _Float16>::type;
      SdT* ws = static_cast<SdT*>(a.dS_chunks) + (sl.item0 + n) * DK * Dv + j0;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) ws[(int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = static_cast<SdT>(accD[R][c][i]);
    }

    // this chunk's dO fragments (zero past the sequence, and on the identity columns and idle waves);
    // the previous chunk's start loading
    using DoF = typename std::conditional<F32IN, f32x4, f16x8>::type;
    DoF dof[NDU][NCT];
    const int Ln = min(C, sl.len - n * C);
#pragma unroll
    for (int u = 0; u < NDU; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int j = 0; j < NDE; ++j) {
          const bool ok = has_do && (SEG || do_row(u, j) < Ln);  // (segmented: zeroed at the load)
          if constexpr (F32IN) dof[u][c][j] = ok ? rdc[u][c][j] : 0.f;
          else dof[u][c][j] = static_cast<_Float16>(ok ? gsc * bf16_bits_to_f32(rdc[u][c][j]) : 0.f);
        }
    if (has_do && n > n_begin) load_do(n - 1, rdx);
    if (active) {

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

    }  // active

    if (NBUF == 1 && n > n_begin) {
      __syncthreads();  // every wave is done reading the single buffer
      dma(recs + (int64_t)(n - 1) * Rec::kBytes, smem);
    }
  };
  // steps in pairs: static buffers and dO registers (see the forward chain's step loop); the segmented
  // kernel's 8-wave workgroups have no registers for the pairs (spills), so it takes one step per
  // iteration with one dO set
  char* const nextA = NBUF == 2 ? smemB : smemA;
  if constexpr (SEG) {
    for (int n = n_end - 1; n >= n_begin; --n) {
      const bool odd = ((n_end - 1 - n) & 1) != 0;
      step(n, odd ? nextA : smemA, odd ? smemA : nextA, rdoA, rdoA);
    }
  } else {
    for (int n = n_end - 1; n >= n_begin; n -= 2) {
      step(n, smemA, nextA, rdoA, rdoB);
      if (n - 1 >= n_begin) step(n - 1, nextA, smemA, rdoB, rdoA);
    }
  }

  if constexpr (SEG) {
    if (sg.mode == kSegMap && active) {
      // entry gradient of a zero-exit segment: N (value columns) or M (identity columns)
      float* dst = ident ? sg.M + segIdx * DK * DK + (j0 - Dv) : sg.N + segIdx * DK * Dv + j0;
      const int ld = ident ? DK : Dv;
#pragma unroll
      for (int R = 0; R < RK; ++R)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * R + 4 * lg + i) * ld + 16 * c + lr] = accD[R][c][i];
      return;
    }
    if (!seg_first || !active) return;
  }
  if (!active) return;  // helper waves
  if (a.dS0) {
    const float inv = 1.f / gsc;  // exact: a power of two
#pragma unroll
    for (int R = 0; R < RK; ++R)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dS0[stBase + (int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] = inv * accD[R][c][i];
  }
}

// ---------------------------------------------------------------------------
// dispatch: NCT column tiles of 16 per wave, NWV column waves per workgroup,
// shaped so that the grid has at least ~256 workgroups when it can
// ---------------------------------------------------------------------------
template <int DK, int C, bool F32IN, int NCT, int NWV>
static hipError_t launch_chain_t(const FwdArgs& a, const char* rec, const float* ut, hipStream_t s) {
  using Cfg = ChainCfg<DK, C, F32IN, NCT, NWV>;
  if constexpr (!Cfg::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    const int ncg = a.Dv / Cfg::kCols;
    const int nbh = seq_items(a.vl, a.B, a.H);
    const int grid = ((nbh + 7) / 8) * 8 * ncg;
    hipLaunchKernelGGL((gdn2_chain_fwd_kernel<DK, C, F32IN, NCT, NWV, false>), dim3(grid), dim3(NWV * kWave), 0, s,
                       a, rec, ut, SegArgs{});
    return hipGetLastError();
  }
}

// Composition of the segment maps: S_in(s+1) = M_s S_in(s) + N_s, S_in(0) = S0
// (or zero), in fp32. One workgroup (4 waves) per (batch*head, 32 value
// columns); the column groups of one head take workgroups 8 apart (one XCD, so
// M_s comes through its L2 once). S_in(s) lives in LDS; each step copies M_s
// into LDS with coalesced loads and forms the product on fp32 matrix cores,
// N_s as the initial accumulator: wave w owns row tiles 2w and 2w+1 (times
// DK / 128) of both 16-column tiles. M_{s+1} and N_{s+1} are loaded into
// registers during step s, so a step waits on no load issued in it (B1 H16
// T64K forward 1.94 -> 1.89 ms; N had been loaded after the next M, so each
// step waited for both).
template <int DK>
// reverse (the backward's exit gradients): S_in(s-1) = M_s S_in(s) + N_s from
// S_in(count-1) = start (dS_final), empty sequences copying start to empty_out (dS0).
// gscale (reverse, 16-bit inputs): start is dS_final, taken times grad_scale() as the reverse chain
// takes it; an empty sequence's dS0 is written without the scale.
__global__ __launch_bounds__(kComposeThreads) void gdn2_seg_compose_kernel(const float* S0, float* S_final, SegArgs sg,
                                                              Varlen vl, int nbh, int H, int Dv, bool reverse,
                                                              const float* gscale) {
  constexpr int LDM = DK + 4, LDS_ = 32 + 4;
  constexpr int NM4 = DK * DK / 4;              // float4 of one M
  constexpr int NT = kComposeThreads, NWC = NT / 64;
  constexpr int MV = (NM4 + NT - 1) / NT;       // per thread
  constexpr int RT = DK / 16;                   // row tiles
  constexpr int RPW = (RT + NWC - 1) / NWC;     // row tiles per wave
  __shared__ __attribute__((aligned(16))) float sM[DK * LDM];
  __shared__ __attribute__((aligned(16))) float sS[DK * LDS_];
  const int ncg = Dv / 32;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int bh = (slot / ncg) * 8 + xcd, j0 = (slot - (slot / ncg) * ncg) * 32;
  if (bh >= nbh) return;  // the grid is rounded up to whole groups of 8
  // this (batch row or sequence, head)'s segments: slots base .. base + count - 1 of M, N, S_in
  int64_t base;
  int count;
  if (vl.cu == nullptr) {
    base = (int64_t)bh * sg.nseg;
    count = sg.nseg;
  } else {
    const int sq = bh / H, h = bh - sq * H;
    base = (int64_t)h * vl.max_segs + vl.seg_first[sq];
    count = vl.seg_first[sq + 1] - vl.seg_first[sq];
  }
  const int tid = threadIdx.x, wid = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const float gsc = grad_scale(gscale, bh);
  for (int e = tid; e < DK * 32; e += NT) {
    const int d = e >> 5, c = e & 31;
    sS[d * LDS_ + c] = S0 ? gsc * S0[((int64_t)bh * DK + d) * Dv + j0 + c] : 0.f;
  }
  float4 mr[MV];
  float nr[RPW][2][4];  // N of the same segment at the lane's accumulator positions
  // step i reads the map of segment src(i) and writes the entry of the next one in walking order
  auto src = [&](int i) { return reverse ? count - 1 - i : i; };
  auto load_m = [&](int s) {
    const float4* M = reinterpret_cast<const float4*>(sg.M + (base + src(s)) * DK * DK);
#pragma unroll
    for (int i = 0; i < MV; ++i)
      if (tid + NT * i < NM4) mr[i] = M[tid + NT * i];
    const float* N = sg.N + (base + src(s)) * DK * Dv + j0;
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int R = wid + NWC * t;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          nr[t][c][i] = R < RT ? N[(int64_t)(16 * R + 4 * lg + i) * Dv + 16 * c + lr] : 0.f;
    }
  };
  if (count == 0) {  // an empty packed sequence has no segment to carry its state: S_final = S0
    __syncthreads();
    for (int e = tid; S_final && e < DK * 32; e += NT) {
      const int d = e >> 5, c = e & 31;
      S_final[((int64_t)bh * DK + d) * Dv + j0 + c] = sS[d * LDS_ + c] / gsc;
    }
    return;
  }
  if (count > 1) load_m(0);
  for (int s = 0; s + 1 < count; ++s) {
    const int64_t sb = base + src(s);
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      const int e = tid + NT * i, row = e / (DK / 4), c4 = 4 * (e % (DK / 4));
      if (e < NM4) *reinterpret_cast<float4*>(sM + row * LDM + c4) = mr[i];
    }
    f32x4 acc[RPW][2];
#pragma unroll
    for (int t = 0; t < RPW; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][c][i] = nr[t][c][i];
    __syncthreads();  // M_s and S_in(s) are in LDS
    if (s + 2 < count) load_m(s + 1);
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int R = wid + NWC * t;
      if (R < RT) {
        for (int k0 = 0; k0 < DK; k0 += 16) {
          const float4 a4 = *reinterpret_cast<const float4*>(sM + (16 * R + lr) * LDM + k0 + 4 * lg);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float* srow = sS + (k0 + 4 * lg + m) * LDS_;
            acc[t][0] = mfma16x16x4(av[m], srow[lr], acc[t][0]);
            acc[t][1] = mfma16x16x4(av[m], srow[16 + lr], acc[t][1]);
          }
        }
      }
    }
    __syncthreads();  // every wave is done reading M_s and S_in(s)
    float* out = sg.S_in + (reverse ? sb - 1 : sb + 1) * DK * Dv + j0;
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int R = wid + NWC * t;
      if (R < RT) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = 16 * R + 4 * lg + i, col = 16 * c + lr;
            sS[d * LDS_ + col] = acc[t][c][i];
            out[(int64_t)d * Dv + col] = acc[t][c][i];
          }
      }
    }
  }
}

// Segment count of the two-level forward: used when the plain chain has too
// few independent column tiles to fill the GPU (and the sizes suit the
// compose kernel: Dv >= 32).
int fwd_segments(int B, int H, int T, int Dk, int Dv, int chunk) {
  if (Dv < 32) return 1;
  const int NC = (T + chunk - 1) / chunk;
  const long nbh = (long)B * H;
  if (nbh * (Dv / 32) >= 512) return 1;     // enough 32-column wave tiles already
  // about one run-pass workgroup per two CUs: with pipelined chain steps, fewer and longer segments cost
  // less than the extra map and composition work of more (B1 H16 d128: T = 8K 0.36 -> 0.31 ms, 16K
  // 0.57 -> 0.52 ms; equal at 32K and 64K; one per CU at 64K was not faster)
  long g = 128 / (nbh * ((Dv + 127) / 128));
  // twice as many where the segments stay at least 64 chunks long (one run-pass workgroup per CU: B1 H16
  // d128 T = 64K 1.67 -> 1.62 ms; at 8K-32K the map and composition work of the shorter segments lost or tied)
  if (g >= 4 && NC / (2 * g) >= 64) g *= 2;
  if (g > NC / 8) g = NC / 8;                // at least 8 chunks per segment
  if (g > 64) g = 64;
  if (g < 4) return 1;
  const int L = (NC + (int)g - 1) / (int)g;
  return (NC + L - 1) / L;                   // segments actually formed
}

size_t fwd_seg_bytes(int B, int H, int T, int Dk, int Dv, int chunk) {
  const int G = fwd_segments(B, H, T, Dk, Dv, chunk);
  if (G <= 1) return 0;
  const size_t nb = (size_t)B * H * G;
  return nb * ((size_t)Dk * Dk + 2 * (size_t)Dk * Dv) * sizeof(float);
}

template <int DK, int C, bool F32IN>
static hipError_t launch_chain_seg(const FwdArgs& a, const char* rec, const float* ut, char* seg, int G,
                                   hipStream_t s) {
  using Cfg = ChainCfg<DK, C, F32IN, 1, kSegWaves>;
  if constexpr (!Cfg::kFits) {
    return hipErrorInvalidConfiguration;
  } else {
    // G segments per (batch row, head) of a dense batch; a packed batch has
    // a.vl.max_segs segment slots per head (from the plan's tables)
    const bool packed = a.vl.cu != nullptr;
    const int NC = (a.T + C - 1) / C, nbh = seq_items(a.vl, a.B, a.H);
    const int64_t slots = packed ? (int64_t)a.H * a.vl.max_segs : (int64_t)nbh * G;
    SegArgs sg;
    sg.nseg = packed ? 0 : G;
    sg.seg_len = packed ? a.vl.seg_len : (NC + G - 1) / G;
    sg.M = reinterpret_cast<float*>(seg);
    sg.N = sg.M + (size_t)slots * DK * DK;
    sg.S_in = sg.N + (size_t)slots * DK * a.Dv;
    const int ncg_map = (a.Dv + DK + Cfg::kCols - 1) / Cfg::kCols, ncg_run = (a.Dv + Cfg::kCols - 1) / Cfg::kCols;
    // (1) maps of every segment but the last of each (batch row or sequence, head)
    sg.mode = kSegMap;
    const int64_t map_items = packed ? slots : (int64_t)nbh * (G - 1);
    hipLaunchKernelGGL((gdn2_chain_fwd_kernel<DK, C, F32IN, 1, kSegWaves, true, 0, true>),
                       dim3(seg_grid(map_items, ncg_map)), dim3(Cfg::kThreads), 0, s, a, rec, ut, sg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (2) entry states of the later segments
    hipLaunchKernelGGL((gdn2_seg_compose_kernel<DK>), dim3(seg_grid(nbh, a.Dv / 32)), dim3(kComposeThreads), 0, s, a.S0,
                       a.S_final, sg, a.vl, nbh, a.H, a.Dv, false, static_cast<const float*>(nullptr));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (3) every segment from its true entry state
    sg.mode = kSegRun;
    hipLaunchKernelGGL((gdn2_chain_fwd_kernel<DK, C, F32IN, 1, kSegWaves, true>), dim3(seg_grid(slots, ncg_run)),
                       dim3(Cfg::kThreads), 0, s, a, rec, ut, sg);
    return hipGetLastError();
  }
}

template <int DK, int C, bool F32IN>
static hipError_t launch_chain_c(const FwdArgs& a, const char* rec, const float* ut, char* seg, hipStream_t s) {
  const int nbh = seq_items(a.vl, a.B, a.H);
  {
    if (a.vl.cu != nullptr) {
      if (seg && a.vl.seg_len > 0) return launch_chain_seg<DK, C, F32IN>(a, rec, ut, seg, 0, s);
    } else {
      const int G = seg ? fwd_segments(a.B, a.H, a.T, DK, a.Dv, C) : 1;
      if (G > 1) return launch_chain_seg<DK, C, F32IN>(a, rec, ut, seg, G, s);
    }
  }
  if (a.Dv == 16) return launch_chain_t<DK, C, F32IN, 1, 1>(a, rec, ut, s);
  // 64 columns per workgroup, over four waves (one per SIMD), from 64 workgroups up (two waves of 32
  // columns: 0.89 -> 0.84 ms for the B8 H16 T4096 training forward); else 32 columns per one-wave
  // workgroup, or 16 for few heads. The two record buffers hold a CU's LDS, so every shape runs one
  // workgroup per CU: narrower workgroups past 256 of them take a second round of the whole walk (B7 H16
  // T4096 training step 2.73 -> 2.03 ms, B3 1.54 -> 1.13 ms with four-wave workgroups from 64 up)
  const int tiles = a.Dv / 32;  // 32-column tiles per head
  if (tiles >= 2 && nbh * (tiles / 2) >= 64) return launch_chain_t<DK, C, F32IN, 1, 4>(a, rec, ut, s);
  if (nbh * tiles >= 256) return launch_chain_t<DK, C, F32IN, 2, 1>(a, rec, ut, s);
  return launch_chain_t<DK, C, F32IN, 1, 1>(a, rec, ut, s);  // few heads: 16 columns per workgroup
}

template <int DK, bool F32IN>
static hipError_t launch_chain_k(const FwdArgs& a, const char* rec, const float* ut, char* seg, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_chain_c<DK, 16, F32IN>(a, rec, ut, seg, s);
    case 32: return launch_chain_c<DK, 32, F32IN>(a, rec, ut, seg, s);
    case 64: return launch_chain_c<DK, 64, F32IN>(a, rec, ut, seg, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_chain_f(const FwdArgs& a, const char* rec, const float* ut, char* seg, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_chain_k<16, F32IN>(a, rec, ut, seg, s);
    case 32: return launch_chain_k<32, F32IN>(a, rec, ut, seg, s);
    case 64: return launch_chain_k<64, F32IN>(a, rec, ut, seg, s);
    case 128: return launch_chain_k<128, F32IN>(a, rec, ut, seg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chain_fwd(const FwdArgs& a, const char* rec, const float* ut, char* seg, hipStream_t s) {
  return a.f32_inputs ? launch_chain_f<true>(a, rec, ut, seg, s) : launch_chain_f<false>(a, rec, ut, seg, s);
}

template <int DK, int C, bool F32IN, int NCT, int NWV>
static hipError_t launch_chain_bwd_t(const BwdArgs& a, const char* rec, hipStream_t s) {
  using Rec = Record<DK, C, F32IN, 1>;
  if constexpr (Rec::kChainBytes > 160 * 1024) {
    return hipErrorInvalidConfiguration;
  } else {
    const int ncg = a.Dv / (16 * NCT * NWV);
    const int nbh = seq_items(a.vl, a.B, a.H);
    const int grid = ((nbh + 7) / 8) * 8 * ncg;
    hipLaunchKernelGGL((gdn2_chain_bwd_kernel<DK, C, F32IN, NCT, NWV, false, kChainHelpers>), dim3(grid),
                       dim3((NWV + kChainHelpers) * kWave), 0, s, a, rec, SegArgs{});
    return hipGetLastError();
  }
}

// The two-level reverse chain: G segments per (batch row, head) of a dense
// batch, or the packed batch's segment slots; seg holds M, N and the composed
// exit gradients (fwd_seg_bytes / varlen_seg_bytes).
template <int DK, int C, bool F32IN>
static hipError_t launch_chain_bwd_seg(const BwdArgs& a, const char* rec, char* seg, int G, hipStream_t s) {
  using Rec = Record<DK, C, F32IN, 1>;
  constexpr int kCols = 16 * kSegWaves;
  if constexpr (Rec::kChainBytes > 160 * 1024) {
    return hipErrorInvalidConfiguration;
  } else {
    const bool packed = a.vl.cu != nullptr;
    const int NC = (a.T + C - 1) / C, nbh = seq_items(a.vl, a.B, a.H);
    const int64_t slots = packed ? (int64_t)a.H * a.vl.max_segs : (int64_t)nbh * G;
    SegArgs sg;
    sg.nseg = packed ? 0 : G;
    sg.seg_len = packed ? a.vl.seg_len : (NC + G - 1) / G;
    sg.M = reinterpret_cast<float*>(seg);
    sg.N = sg.M + (size_t)slots * DK * DK;
    sg.S_in = sg.N + (size_t)slots * DK * a.Dv;
    const int ncg_map = (a.Dv + DK + kCols - 1) / kCols, ncg_run = (a.Dv + kCols - 1) / kCols;
    // (1) maps of every segment but the first of each (batch row or sequence, head)
    sg.mode = kSegMap;
    const int64_t map_items = packed ? slots : (int64_t)nbh * (G - 1);
    hipLaunchKernelGGL((gdn2_chain_bwd_kernel<DK, C, F32IN, 1, kSegWaves, true>), dim3(seg_grid(map_items, ncg_map)),
                       dim3(kSegWaves * kWave), 0, s, a, rec, sg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (2) exit gradients of the earlier segments, composed backwards from dS_final
    hipLaunchKernelGGL((gdn2_seg_compose_kernel<DK>), dim3(seg_grid(nbh, a.Dv / 32)), dim3(kComposeThreads), 0, s, a.dS_final,
                       a.dS0, sg, a.vl, nbh, a.H, a.Dv, true, a.gscale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (3) every segment from its true exit gradient
    sg.mode = kSegRun;
    hipLaunchKernelGGL((gdn2_chain_bwd_kernel<DK, C, F32IN, 1, kSegWaves, true>), dim3(seg_grid(slots, ncg_run)),
                       dim3(kSegWaves * kWave), 0, s, a, rec, sg);
    return hipGetLastError();
  }
}

template <int DK, int C, bool F32IN>
static hipError_t launch_chain_bwd_c(const BwdArgs& a, const char* rec, char* seg, hipStream_t s) {
  const int nbh = seq_items(a.vl, a.B, a.H);
  if (a.vl.cu != nullptr) {
    if (seg && a.vl.seg_len > 0) return launch_chain_bwd_seg<DK, C, F32IN>(a, rec, seg, 0, s);
  } else {
    const int G = seg ? fwd_segments(a.B, a.H, a.T, DK, a.Dv, C) : 1;
    if (G > 1) return launch_chain_bwd_seg<DK, C, F32IN>(a, rec, seg, G, s);
  }
  if (a.Dv == 16) return launch_chain_bwd_t<DK, C, F32IN, 1, 1>(a, rec, s);
  // workgroup shapes as in the forward chain (four waves of 16 columns: 1.44 -> 1.39 ms for the B8 H16
  // T4096 backward), plus the helper waves
  const int tiles = a.Dv / 32;
  if (tiles >= 2 && nbh * (tiles / 2) >= 64) return launch_chain_bwd_t<DK, C, F32IN, 1, 4>(a, rec, s);
  if (nbh * tiles >= 256) return launch_chain_bwd_t<DK, C, F32IN, 2, 1>(a, rec, s);
  return launch_chain_bwd_t<DK, C, F32IN, 1, 1>(a, rec, s);
}

template <int DK, bool F32IN>
static hipError_t launch_chain_bwd_k(const BwdArgs& a, const char* rec, char* seg, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_chain_bwd_c<DK, 16, F32IN>(a, rec, seg, s);
    case 32: return launch_chain_bwd_c<DK, 32, F32IN>(a, rec, seg, s);
    case 64: return launch_chain_bwd_c<DK, 64, F32IN>(a, rec, seg, s);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
static hipError_t launch_chain_bwd_f(const BwdArgs& a, const char* rec, char* seg, hipStream_t s) {
  switch (a.Dk) {
    case 16: return launch_chain_bwd_k<16, F32IN>(a, rec, seg, s);
    case 32: return launch_chain_bwd_k<32, F32IN>(a, rec, seg, s);
    case 64: return launch_chain_bwd_k<64, F32IN>(a, rec, seg, s);
    case 128: return launch_chain_bwd_k<128, F32IN>(a, rec, seg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chain_bwd(const BwdArgs& a, const char* rec, char* seg, hipStream_t s) {
  return a.f32_inputs ? launch_chain_bwd_f<true>(a, rec, seg, s) : launch_chain_bwd_f<false>(a, rec, seg, s);
}

}  // namespace gdn2
