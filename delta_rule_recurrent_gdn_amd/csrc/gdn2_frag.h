// gdn2_frag.h -- matrix-core operand fragments and the per-chunk record layout
// shared by the chunk-parallel preparation kernels and the sequential chain
// kernels (gfx950, wave64).
//
// Fragment. A "unit" is the left operand of one matrix-core step for a 16-row
// tile: 16 rows x KU contraction indices, 64 lanes x 16 bytes = 1 KB, lane l at
// byte 16*l. Lane l holds row (l % 16) and the contraction slots of lane group
// g = l / 16:
//   16-bit operands (KU = 32, v_mfma_f32_16x16x32_f16): slot j < 4 is index
//     4g + j, slot j >= 4 is index 16 + 4g + (j - 4);
//   fp32 operands (KU = 16, four v_mfma_f32_16x16x4_f32): slot j is 4g + j.
// An fp32 accumulator tile holds rows 4g + i of column (l % 16), so the right
// operand of one unit is exactly the accumulators of the 16-row tiles 2u and
// 2u+1 (16-bit; slots j < 4 from the first, j >= 4 from the second) or of tile
// u (fp32; step i uses accumulator element i). A product whose right operand
// is a running state or write matrix therefore never stages it through LDS,
// and the left operand is read with one 16-byte access per lane.
//
// Record. The chunk-parallel kernels store, per (batch*head, chunk), the left
// operands the chain needs as consecutive units (row tile major, then unit),
// followed by one unit holding exp(g_C) per key channel (and, in the backward
// record, the operands of the per-chunk gradient kernel).
#pragma once

#include "gdn2_common.h"

namespace gdn2 {

template <bool F32IN>
struct Frag {
  using OpT = typename std::conditional<F32IN, float, _Float16>::type;
  static constexpr int KU = F32IN ? 16 : 32;      // contraction indices per unit
  static constexpr int kUnitBytes = 1024;
  // contraction index of slot j in lane group g
  __device__ __forceinline__ static int kslot(int g, int j) {
    if constexpr (F32IN) return 4 * g + j;
    else return j < 4 ? 4 * g + j : 12 + 4 * g + j;
  }
  static constexpr int units(int K) { return (K + KU - 1) / KU; }
};

// Per-chunk record: matrices in units and the exp(g_C) unit.
// Forward (DIR = 0):  Wn = -W [C x DK], Qs = q exp(g) [C x DK],
//                     KbT = (k exp(g_C - g))^T [DK x C], P [C x C], then exp(g_C).
// Backward (DIR = 1): PT = P^T [C x C], Kb [C x DK], QsT [DK x C], WnT = -W^T [DK x C],
//                     exp(g_C), then T = (I + A)^-1 [C x C] and Kh = b k exp(g) [C x DK].
// The sequential chains read only the leading kChainUnits units (T and Kh are
// for the per-chunk gradient kernel), so they copy a contiguous prefix.
template <int DK, int C, bool F32IN, int DIR>
struct Record {
  using F = Frag<F32IN>;
  static constexpr int UK = F::units(DK), UC = F::units(C);
  static constexpr int RC = C / 16, RK = DK / 16;  // 16-row tiles
  // unit offsets of the matrices
  static constexpr int u0 = 0;
  static constexpr int u1 = u0 + (DIR == 0 ? RC * UK : RC * UC);
  static constexpr int u2 = u1 + RC * UK;
  static constexpr int u3 = u2 + RK * UC;
  static constexpr int uG = u3 + (DIR == 0 ? RC * UC : RK * UC);
  static constexpr int kChainUnits = uG + 1;
  static constexpr int u4 = kChainUnits;           // DIR 1 only
  static constexpr int u5 = u4 + RC * UC;          // DIR 1 only
  static constexpr int kUnits = DIR == 0 ? kChainUnits : u5 + RC * UK;
  static constexpr int kBytes = kUnits * F::kUnitBytes;
  static constexpr int kChainBytes = kChainUnits * F::kUnitBytes;
  static_assert(DK * 4 <= 1024, "exp(g_C) must fit one unit");
};

// Byte offset of the wide-decay flag of a record (gdn2_wide.h): the last word of the exp(g_C)
// unit, which uses its first DK floats only. The fast record pass writes it for every chunk it
// covers (1: the chunk's record comes from the wide pass instead).
template <class R>
__host__ __device__ constexpr int wide_flag_offset() {
  return R::uG * 1024 + 1020;
}

// Write the units of a row-major matrix X [M][K] (operand type, leading
// dimension ld, in LDS) to dst (global): unit (R, u) at dst + (R * units(K) + u) KB.
// Units are dealt round-robin to the nw waves starting at wave w0.
template <bool F32IN>
__device__ __forceinline__ void write_units(const typename Frag<F32IN>::OpT* X, int ld, int M, int K, char* dst,
                                            int wid, int nw) {
  using F = Frag<F32IN>;
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int nu = F::units(K), total = (M / 16) * nu;
  for (int t = wid; t < total; t += nw) {
    const int R = t / nu, u = t - R * nu;
    const int k0 = F::KU * u;
    const auto* row = X + (16 * R + r) * ld;
    uint4 out;
    if constexpr (F32IN) {
      const float4 v = *reinterpret_cast<const float4*>(row + k0 + 4 * g);
      out = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w));
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(row + k0 + 4 * g);
      uint2 b = make_uint2(0u, 0u);
      if (k0 + 16 < K) b = *reinterpret_cast<const uint2*>(row + k0 + 16 + 4 * g);
      out = make_uint4(a.x, a.y, b.x, b.y);
    }
    *reinterpret_cast<uint4*>(dst + (int64_t)t * F::kUnitBytes + 16 * l) = out;
  }
}

// Same for an fp32 matrix in LDS, rounded to the operand type on the way.
template <bool F32IN>
__device__ __forceinline__ void write_units_f32(const float* X, int ld, int M, int K, char* dst, int wid, int nw) {
  using F = Frag<F32IN>;
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int nu = F::units(K), total = (M / 16) * nu;
  for (int t = wid; t < total; t += nw) {
    const int R = t / nu, u = t - R * nu;
    const int k0 = F::KU * u;
    const float* row = X + (16 * R + r) * ld;
    uint4 out;
    if constexpr (F32IN) {
      const float4 v = *reinterpret_cast<const float4*>(row + k0 + 4 * g);
      out = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w));
    } else {
      f16x8 h;
      const float4 a = *reinterpret_cast<const float4*>(row + k0 + 4 * g);
      float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k0 + 16 < K) b = *reinterpret_cast<const float4*>(row + k0 + 16 + 4 * g);
      h[0] = static_cast<_Float16>(a.x); h[1] = static_cast<_Float16>(a.y);
      h[2] = static_cast<_Float16>(a.z); h[3] = static_cast<_Float16>(a.w);
      h[4] = static_cast<_Float16>(b.x); h[5] = static_cast<_Float16>(b.y);
      h[6] = static_cast<_Float16>(b.z); h[7] = static_cast<_Float16>(b.w);
      out = __builtin_bit_cast(uint4, h);
    }
    *reinterpret_cast<uint4*>(dst + (int64_t)t * F::kUnitBytes + 16 * l) = out;
  }
}

// Unpack unit (R, u) of a record matrix [M][K] into row-major LDS copies:
// X[row][k] (ldx) and, when XT is not null, XT[k][row] (ldt); indices past K skipped.
// VEC: X's row takes the lane's slots as runs of 4 consecutive contraction indices, one vector store
// each, instead of one store per element.
template <bool F32IN, bool VEC, typename OpT>
__device__ __forceinline__ void unpack_unit(const uint4& v, int R, int u, int K, OpT* X, int ldx, OpT* XT, int ldt) {
  using F = Frag<F32IN>;
  const int l = lane_id(), r = 16 * R + (l & 15), g = l >> 4;
  if constexpr (F32IN) {
    const float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
    if constexpr (VEC) *reinterpret_cast<uint4*>(X + r * ldx + F::KU * u + F::kslot(g, 0)) = v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = F::KU * u + F::kslot(g, j);
      if constexpr (!VEC) X[r * ldx + k] = x[j];
      if (XT) XT[k * ldt + r] = x[j];
    }
  } else {
    const f16x8 h = __builtin_bit_cast(f16x8, v);
    if constexpr (VEC) {  // slots 0-3 and 4-7; K is a multiple of 16, so a run lies wholly below K or not
      const int k0 = F::KU * u + F::kslot(g, 0), k1 = F::KU * u + F::kslot(g, 4);
      if (k0 < K) *reinterpret_cast<uint2*>(X + r * ldx + k0) = make_uint2(v.x, v.y);
      if (k1 < K) *reinterpret_cast<uint2*>(X + r * ldx + k1) = make_uint2(v.z, v.w);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = F::KU * u + F::kslot(g, j);
      if (k < K) {
        if constexpr (!VEC) X[r * ldx + k] = h[j];
        if (XT) XT[k * ldt + r] = h[j];
      }
    }
  }
}

// Right operand of unit u from accumulator tiles (16-bit: tiles 2u, 2u+1).
__device__ __forceinline__ f16x8 rhs_from_acc(const f32x4& t0, const f32x4& t1) {
  f16x8 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[i] = static_cast<_Float16>(t0[i]);
    b[4 + i] = static_cast<_Float16>(t1[i]);
  }
  return b;
}

// acc += unit(A) * rhs, 16-bit.
__device__ __forceinline__ void unit_mma(f32x4& acc, const uint4& a, const f16x8& b) {
  acc = mfma16x16x32(__builtin_bit_cast(f16x8, a), b, acc);
}
// acc += unit(A) * rhs, fp32: the right operand is the accumulator tile itself.
__device__ __forceinline__ void unit_mma(f32x4& acc, const uint4& a, const f32x4& b) {
  acc = mfma16x16x4(__uint_as_float(a.x), b[0], acc);
  acc = mfma16x16x4(__uint_as_float(a.y), b[1], acc);
  acc = mfma16x16x4(__uint_as_float(a.z), b[2], acc);
  acc = mfma16x16x4(__uint_as_float(a.w), b[3], acc);
}

// acc + x y^T over four contraction indices per lane group, fp32 operands
// (both taken in the same lane-slot order).
__device__ __forceinline__ f32x4 unit_mma_ff(f32x4 acc, const f32x4& x, const f32x4& y) {
  acc = mfma16x16x4(x[0], y[0], acc);
  acc = mfma16x16x4(x[1], y[1], acc);
  acc = mfma16x16x4(x[2], y[2], acc);
  acc = mfma16x16x4(x[3], y[3], acc);
  return acc;
}

}  // namespace gdn2
