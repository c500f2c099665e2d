// gdn2_common.h -- device helpers shared by the GDN-2 kernels (gfx950, wave64).
//
// Matrix-core tiles are 16x16 with fp32 accumulators. For every
// v_mfma_f32_16x16xK instruction used here, lane l of the wave supplies row
// (l % 16) of the left operand and column (l % 16) of the right operand, with
// a contiguous group of K/4 contraction indices selected by (l / 16); the
// accumulator holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3. The two
// operands always take their contraction indices from the same lane slot, so
// the products below only rely on that row/column assignment and on the
// accumulator layout.
//
// Accumulation chains never mix instruction shapes: a contraction remainder of
// 16 is issued as a 16x16x32 product with the upper half of K zeroed (lane
// groups 2 and 3 contribute zeros), so every product accumulating into one
// register tile is the same instruction. (A 16x16x16 product feeding a
// 16x16x32 product's accumulator input back-to-back gave wrong results on
// gfx950 with the compiler's instruction spacing.)
//
// Operands staged in LDS are stored "K-contiguous": a left operand X as
// [M][K] and a right operand as [N][K] (its transpose), both row-major with a
// padded leading dimension, so every lane reads its contraction group with one
// vector load. C(16x16) += X(16xK) * Y(16xK)^T is the basic tile product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on the gfx9 family (gfx950 included): 32-bit
// data format, no swizzle, so offsets are plain byte offsets; accesses past
// num_records read zero and are not written.
constexpr int kBufferRsrcWord3 = 0x00020000;

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------------------
// storage conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Gate front end (pre-activation inputs): b = sigmoid(b_raw), w = sigmoid(w_raw),
// log_alpha = -softplus(a_raw) = -log(1 + exp(a_raw)), in fp32.
// Hardware exp2 / log2 / reciprocal forms (about 1 ulp each). -softplus is
// taken as -(max(x, 0) + log(1 + exp(-|x|))), which never overflows; its
// absolute error stays below 1e-7, also where the result is tiny.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float neg_softplus_f(float x) {
  return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x))));
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ float bf16_to_f32(__bf16 h) { return static_cast<float>(h); }

// Load 8 consecutive inputs of storage type (fp32 or bf16) as fp32.
template <bool F32IN>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&out)[8]) {
  if constexpr (F32IN) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Load 4 consecutive inputs as fp32.
template <bool F32IN>
__device__ __forceinline__ void load4(const void* base, int64_t idx, float (&out)[4]) {
  if constexpr (F32IN) {
    float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xffff0000u);
  }
}

// Guarded element load without a branch: reads element idx when ok, else the
// always-valid element safe, and returns zero when not ok. A run of these stays
// in flight together (a load inside an if-block makes the compiler wait for it
// at the end of the block).
template <typename T>
__device__ __forceinline__ T ld_sel(const T* p, int64_t idx, int64_t safe, bool ok) {
  const T v = p[ok ? idx : safe];
  return ok ? v : T(0);
}

template <bool F32IN>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (F32IN) return static_cast<const float*>(base)[idx];
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
}

// load1 with ld_sel's guard: zero when !ok, reading the always-valid element safe.
template <bool F32IN>
__device__ __forceinline__ float load1_sel(const void* base, int64_t idx, int64_t safe, bool ok) {
  if constexpr (F32IN) return ld_sel(static_cast<const float*>(base), idx, safe, ok);
  else return bf16_bits_to_f32(ld_sel(static_cast<const uint16_t*>(base), idx, safe, ok));
}

// Raw register copies of 4 / 8 consecutive inputs in their storage type, so a
// chunk's inputs can be fetched from HBM one chunk ahead of their use.
template <bool F32IN> struct Raw4 { uint2 u; };
template <> struct Raw4<true> { float4 f; };
template <bool F32IN> struct Raw8 { uint4 u; };
template <> struct Raw8<true> { float4 f0, f1; };

template <bool F32IN>
__device__ __forceinline__ void ld_raw(Raw4<F32IN>& r, const void* base, int64_t idx) {
  if constexpr (F32IN) r.f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  else r.u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
}
// Gates of one value per (token, head) ([., T, H] layout): the value at sidx
// broadcast to every channel. These load the channels of a gate in either layout.
template <bool F32IN>
__device__ __forceinline__ void ld_raw_gate(Raw4<F32IN>& r, const void* base, int64_t idx, int64_t sidx, bool scalar) {
  if (!scalar) {
    ld_raw(r, base, idx);
  } else if constexpr (F32IN) {
    const float x = static_cast<const float*>(base)[sidx];
    r.f = make_float4(x, x, x, x);
  } else {
    uint32_t x = static_cast<const uint16_t*>(base)[sidx];
    x |= x << 16;
    r.u = make_uint2(x, x);
  }
}
template <bool F32IN>
__device__ __forceinline__ void load4_gate(const void* base, int64_t idx, int64_t sidx, bool scalar, float (&out)[4]) {
  if (!scalar) {
    load4<F32IN>(base, idx, out);
  } else {
    const float x = load1<F32IN>(base, sidx);
    out[0] = out[1] = out[2] = out[3] = x;
  }
}
template <bool F32IN>
__device__ __forceinline__ void load8_gate(const void* base, int64_t idx, int64_t sidx, bool scalar, float (&out)[8]) {
  if (!scalar) {
    load8<F32IN>(base, idx, out);
  } else {
    const float x = load1<F32IN>(base, sidx);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = x;
  }
}
__device__ __forceinline__ float4 load_la4(const float* base, int64_t idx, int64_t sidx, bool scalar) {
  if (!scalar) return *reinterpret_cast<const float4*>(base + idx);
  const float x = base[sidx];
  return make_float4(x, x, x, x);
}

template <bool F32IN>
__device__ __forceinline__ void ld_raw(Raw8<F32IN>& r, const void* base, int64_t idx) {
  if constexpr (F32IN) {
    r.f0 = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    r.f1 = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx + 4);
  } else {
    r.u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  }
}
template <bool F32IN>
__device__ __forceinline__ void ld_raw_gate(Raw8<F32IN>& r, const void* base, int64_t idx, int64_t sidx, bool scalar) {
  if (!scalar) {
    ld_raw(r, base, idx);
  } else if constexpr (F32IN) {
    const float x = static_cast<const float*>(base)[sidx];
    r.f0 = r.f1 = make_float4(x, x, x, x);
  } else {
    uint32_t x = static_cast<const uint16_t*>(base)[sidx];
    x |= x << 16;
    r.u = make_uint4(x, x, x, x);
  }
}
template <bool F32IN>
__device__ __forceinline__ void zero_raw(Raw4<F32IN>& r) {
  if constexpr (F32IN) r.f = make_float4(0.f, 0.f, 0.f, 0.f);
  else r.u = make_uint2(0u, 0u);
}
template <bool F32IN>
__device__ __forceinline__ void zero_raw(Raw8<F32IN>& r) {
  if constexpr (F32IN) r.f0 = r.f1 = make_float4(0.f, 0.f, 0.f, 0.f);
  else r.u = make_uint4(0u, 0u, 0u, 0u);
}
template <bool F32IN>
__device__ __forceinline__ void cvt(const Raw4<F32IN>& r, float (&o)[4]) {
  if constexpr (F32IN) {
    o[0] = r.f.x; o[1] = r.f.y; o[2] = r.f.z; o[3] = r.f.w;
  } else {
    o[0] = __uint_as_float(r.u.x << 16); o[1] = __uint_as_float(r.u.x & 0xffff0000u);
    o[2] = __uint_as_float(r.u.y << 16); o[3] = __uint_as_float(r.u.y & 0xffff0000u);
  }
}
template <bool F32IN>
__device__ __forceinline__ void cvt(const Raw8<F32IN>& r, float (&o)[8]) {
  if constexpr (F32IN) {
    o[0] = r.f0.x; o[1] = r.f0.y; o[2] = r.f0.z; o[3] = r.f0.w;
    o[4] = r.f1.x; o[5] = r.f1.y; o[6] = r.f1.z; o[7] = r.f1.w;
  } else {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Store 4 consecutive values of type T (8 bytes for 16-bit T, 16 bytes for fp32).
template <typename T>
__device__ __forceinline__ void st4(T* dst, float a0, float a1, float a2, float a3) {
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 v;
    v[0] = static_cast<T>(a0); v[1] = static_cast<T>(a1); v[2] = static_cast<T>(a2); v[3] = static_cast<T>(a3);
    *reinterpret_cast<v4*>(dst) = v;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(a0, a1, a2, a3);
  }
}

// ---------------------------------------------------------------------------
// matrix-core primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// C += X(16xK) Y(16xK)^T with X, Y in LDS, K-contiguous rows; K % 16 == 0.
// T = _Float16 or __bf16 (16-bit matrix-core operands) or float (fp32 matrix cores).
template <typename T>
__device__ __forceinline__ void mma_nt(f32x4& acc, const T* X, int ldx, const T* Y, int ldy, int K) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (sizeof(T) == 2) {
    typedef T v8 __attribute__((ext_vector_type(8)));
    typedef T v4 __attribute__((ext_vector_type(4)));
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
      const v8 a = *reinterpret_cast<const v8*>(X + r * ldx + k0 + 8 * g);
      const v8 b = *reinterpret_cast<const v8*>(Y + r * ldy + k0 + 8 * g);
      acc = mfma16x16x32(a, b, acc);
    }
    if (k0 < K) {
      v8 a = {}, b = {};
      if (g < 2) {
        a = *reinterpret_cast<const v8*>(X + r * ldx + k0 + 8 * g);
        b = *reinterpret_cast<const v8*>(Y + r * ldy + k0 + 8 * g);
      }
      acc = mfma16x16x32(a, b, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 4) acc = mfma16x16x4(X[r * ldx + k0 + g], Y[r * ldy + k0 + g], acc);
  }
}

// Compile-time-K variant (fully unrolled).
template <int K, typename T>
__device__ __forceinline__ void mma_nt_k(f32x4& acc, const T* X, int ldx, const T* Y, int ldy) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (sizeof(T) == 2) {
    typedef T v8 __attribute__((ext_vector_type(8)));
    typedef T v4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
      const v8 a = *reinterpret_cast<const v8*>(X + r * ldx + k0 + 8 * g);
      const v8 b = *reinterpret_cast<const v8*>(Y + r * ldy + k0 + 8 * g);
      acc = mfma16x16x32(a, b, acc);
    }
    if constexpr (K % 32 == 16) {
      v8 a = {}, b = {};
      if (g < 2) {
        a = *reinterpret_cast<const v8*>(X + r * ldx + (K - 16) + 8 * g);
        b = *reinterpret_cast<const v8*>(Y + r * ldy + (K - 16) + 8 * g);
      }
      acc = mfma16x16x32(a, b, acc);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) acc = mfma16x16x4(X[r * ldx + k0 + g], Y[r * ldy + k0 + g], acc);
  }
}

// Split product for wide-range operands: X = Xh + Xl, Y = Yh + Yl (bf16 pairs);
// C += Xh Yh^T + Xh Yl^T + Xl Yh^T  (the Xl Yl^T term is below fp32 rounding).
template <int K>
__device__ __forceinline__ void mma_nt_split_k(f32x4& acc, const __bf16* Xh, const __bf16* Xl, int ldx,
                                               const __bf16* Yh, const __bf16* Yl, int ldy) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    const int ox = r * ldx + k0 + 8 * g, oy = r * ldy + k0 + 8 * g;
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Xh + ox);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(Xl + ox);
    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Yh + oy);
    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Yl + oy);
    acc = mfma16x16x32(al, bh, acc);
    acc = mfma16x16x32(ah, bl, acc);
    acc = mfma16x16x32(ah, bh, acc);
  }
  if constexpr (K % 32 == 16) {
    bf16x8 ah = {}, al = {}, bh = {}, bl = {};
    if (g < 2) {
      const int ox = r * ldx + (K - 16) + 8 * g, oy = r * ldy + (K - 16) + 8 * g;
      ah = *reinterpret_cast<const bf16x8*>(Xh + ox);
      al = *reinterpret_cast<const bf16x8*>(Xl + ox);
      bh = *reinterpret_cast<const bf16x8*>(Yh + oy);
      bl = *reinterpret_cast<const bf16x8*>(Yl + oy);
    }
    acc = mfma16x16x32(al, bh, acc);
    acc = mfma16x16x32(ah, bl, acc);
    acc = mfma16x16x32(ah, bh, acc);
  }
}

// C += X Y^T where X and Y are fp32 in LDS, converted on load to the operand
// type T. Y is read either K-contiguous ([N][K], YT=true) or as [K][N]
// (YT=false). Used for the small triangular products; K % 16 == 0.
template <typename T, bool YT>
__device__ __forceinline__ void mma_f32src(f32x4& acc, const float* X, int ldx, const float* Y, int ldy, int K) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    for (int k0 = 0; k0 < K; k0 += 16) {
      v4 a, b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + 4 * g + i;
        a[i] = static_cast<T>(X[r * ldx + k]);
        b[i] = static_cast<T>(YT ? Y[r * ldy + k] : Y[k * ldy + r]);
      }
      acc = mfma16x16x16(a, b, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 4) {
      const int k = k0 + g;
      acc = mfma16x16x4(X[r * ldx + k], YT ? Y[r * ldy + k] : Y[k * ldy + r], acc);
    }
  }
}

// C += X Y^T with X 16-bit in LDS (K-contiguous) and Y fp32 in LDS K-contiguous,
// converted on load. K % 16 == 0.
template <typename T>
__device__ __forceinline__ void mma_nt_yf32(f32x4& acc, const T* X, int ldx, const float* Y, int ldy, int K) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (sizeof(T) == 2) {
    typedef T v8 __attribute__((ext_vector_type(8)));
    typedef T v4 __attribute__((ext_vector_type(4)));
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
      const v8 a = *reinterpret_cast<const v8*>(X + r * ldx + k0 + 8 * g);
      const float4 y0 = *reinterpret_cast<const float4*>(Y + r * ldy + k0 + 8 * g);
      const float4 y1 = *reinterpret_cast<const float4*>(Y + r * ldy + k0 + 8 * g + 4);
      v8 b;
      b[0] = static_cast<T>(y0.x); b[1] = static_cast<T>(y0.y); b[2] = static_cast<T>(y0.z); b[3] = static_cast<T>(y0.w);
      b[4] = static_cast<T>(y1.x); b[5] = static_cast<T>(y1.y); b[6] = static_cast<T>(y1.z); b[7] = static_cast<T>(y1.w);
      acc = mfma16x16x32(a, b, acc);
    }
    if (k0 < K) {
      v8 a = {}, b = {};
      if (g < 2) {
        a = *reinterpret_cast<const v8*>(X + r * ldx + k0 + 8 * g);
        const float4 y0 = *reinterpret_cast<const float4*>(Y + r * ldy + k0 + 8 * g);
        const float4 y1 = *reinterpret_cast<const float4*>(Y + r * ldy + k0 + 8 * g + 4);
        b[0] = static_cast<T>(y0.x); b[1] = static_cast<T>(y0.y); b[2] = static_cast<T>(y0.z); b[3] = static_cast<T>(y0.w);
        b[4] = static_cast<T>(y1.x); b[5] = static_cast<T>(y1.y); b[6] = static_cast<T>(y1.z); b[7] = static_cast<T>(y1.w);
      }
      acc = mfma16x16x32(a, b, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 4) acc = mfma16x16x4(X[r * ldx + k0 + g], Y[r * ldy + k0 + g], acc);
  }
}

// Same with X fp32 (converted) and Y 16-bit. A 16-bit Y may hold each row's 8-element blocks permuted:
// block b of row srow0 + r stored at block b ^ (((srow0 + r) / 8) & smask) (smask 0: plain rows).
template <typename T>
__device__ __forceinline__ void mma_nt_xf32(f32x4& acc, const float* X, int ldx, const T* Y, int ldy, int K,
                                            int srow0 = 0, int smask = 0) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (sizeof(T) == 2) {
    const int sw = 8 * (((srow0 + r) >> 3) & smask);
    typedef T v8 __attribute__((ext_vector_type(8)));
    typedef T v4 __attribute__((ext_vector_type(4)));
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
      const float4 x0 = *reinterpret_cast<const float4*>(X + r * ldx + k0 + 8 * g);
      const float4 x1 = *reinterpret_cast<const float4*>(X + r * ldx + k0 + 8 * g + 4);
      v8 a;
      a[0] = static_cast<T>(x0.x); a[1] = static_cast<T>(x0.y); a[2] = static_cast<T>(x0.z); a[3] = static_cast<T>(x0.w);
      a[4] = static_cast<T>(x1.x); a[5] = static_cast<T>(x1.y); a[6] = static_cast<T>(x1.z); a[7] = static_cast<T>(x1.w);
      const v8 b = *reinterpret_cast<const v8*>(Y + r * ldy + ((k0 + 8 * g) ^ sw));
      acc = mfma16x16x32(a, b, acc);
    }
    if (k0 < K) {
      v8 a = {}, b = {};
      if (g < 2) {
        const float4 x0 = *reinterpret_cast<const float4*>(X + r * ldx + k0 + 8 * g);
        const float4 x1 = *reinterpret_cast<const float4*>(X + r * ldx + k0 + 8 * g + 4);
        a[0] = static_cast<T>(x0.x); a[1] = static_cast<T>(x0.y); a[2] = static_cast<T>(x0.z); a[3] = static_cast<T>(x0.w);
        a[4] = static_cast<T>(x1.x); a[5] = static_cast<T>(x1.y); a[6] = static_cast<T>(x1.z); a[7] = static_cast<T>(x1.w);
        b = *reinterpret_cast<const v8*>(Y + r * ldy + ((k0 + 8 * g) ^ sw));
      }
      acc = mfma16x16x32(a, b, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 4) acc = mfma16x16x4(X[r * ldx + k0 + g], Y[r * ldy + k0 + g], acc);
  }
}

// ---------------------------------------------------------------------------
// accumulator tile stores (lane holds rows 4*(l/16)+i, column l%16)
// ---------------------------------------------------------------------------
// Row-major store of a tile into an LDS/global matrix [rows][ld] of type T.
template <typename T>
__device__ __forceinline__ void store_tile(T* dst, int ld, const f32x4& acc, float scale = 1.f) {
  const int l = lane_id();
  const int c = l & 15, r0 = 4 * (l >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(r0 + i) * ld + c] = static_cast<T>(scale * acc[i]);
}

// Transposed store: dst[col][row] so the 4 rows of a lane are contiguous.
template <typename T>
__device__ __forceinline__ void store_tile_t(T* dst, int ld, const f32x4& acc, float scale = 1.f) {
  const int l = lane_id();
  const int c = l & 15, r0 = 4 * (l >> 4);
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = static_cast<T>(scale * acc[i]);
    *reinterpret_cast<v4*>(dst + c * ld + r0) = v;
  } else {
    *reinterpret_cast<float4*>(dst + c * ld + r0) =
        make_float4(scale * acc[0], scale * acc[1], scale * acc[2], scale * acc[3]);
  }
}

// ---------------------------------------------------------------------------
// (I + A)^-1 of one strictly lower triangular 16x16 block, by one wave.
//
// A is nilpotent (A^16 = 0), so (I + A)^-1 = sum_{j=0}^{15} (-A)^j, evaluated
// by the Horner recursion X <- I - A X (15 steps, starting from X = I). A stays
// in registers in the left-operand layout; the accumulator layout of a 16x16
// product is the right-operand layout (lane holds rows 4*(l/16)+i of column
// l%16), so X never leaves registers. With 16-bit operands X is carried as an
// fp16 hi/lo pair (two products per step) so that its rounding does not build
// up over the 15 steps. On return the block at Ab (fp32, leading dimension
// ld) holds (I + A)^-1, including its zero upper triangle.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void invert_unit_lower16(float* Ab, int ld) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  f32x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (4 * g + i == r) ? 1.f : 0.f;
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = static_cast<T>(Ab[r * ld + 4 * g + i]);
#pragma unroll 1
    for (int step = 0; step < 15; ++step) {
      v4 xh, xl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xh[i] = static_cast<T>(x[i]);
        xl[i] = static_cast<T>(x[i] - static_cast<float>(xh[i]));
      }
      f32x4 d = zero4();
      d = mfma16x16x16(a, xl, d);
      d = mfma16x16x16(a, xh, d);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = ((4 * g + i == r) ? 1.f : 0.f) - d[i];
    }
  } else {
    // fp32 matrix cores: product j pairs lane group g with contraction index 4g+j,
    // which is exactly the row this lane holds in x[j]
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = Ab[r * ld + 4 * g + j];
#pragma unroll 1
    for (int step = 0; step < 15; ++step) {
      f32x4 d = zero4();
#pragma unroll
      for (int j = 0; j < 4; ++j) d = mfma16x16x4(a[j], x[j], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = ((4 * g + i == r) ? 1.f : 0.f) - d[i];
    }
  }
  // all lanes have read A before any lane overwrites the block (one wave, in order)
  store_tile(Ab, ld, x);
}

// Runtime-K split product (K % 16 == 0): C += Xh Yh^T + Xh Yl^T + Xl Yh^T, bf16 pairs.
__device__ __forceinline__ void mma_nt_split(f32x4& acc, const __bf16* Xh, const __bf16* Xl, int ldx,
                                             const __bf16* Yh, const __bf16* Yl, int ldy, int K) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  int k0 = 0;
  for (; k0 + 32 <= K; k0 += 32) {
    const int ox = r * ldx + k0 + 8 * g, oy = r * ldy + k0 + 8 * g;
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Xh + ox);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(Xl + ox);
    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Yh + oy);
    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Yl + oy);
    acc = mfma16x16x32(al, bh, acc);
    acc = mfma16x16x32(ah, bl, acc);
    acc = mfma16x16x32(ah, bh, acc);
  }
  if (k0 < K) {
    bf16x8 ah = {}, al = {}, bh = {}, bl = {};
    if (g < 2) {
      const int ox = r * ldx + k0 + 8 * g, oy = r * ldy + k0 + 8 * g;
      ah = *reinterpret_cast<const bf16x8*>(Xh + ox);
      al = *reinterpret_cast<const bf16x8*>(Xl + ox);
      bh = *reinterpret_cast<const bf16x8*>(Yh + oy);
      bl = *reinterpret_cast<const bf16x8*>(Yl + oy);
    }
    acc = mfma16x16x32(al, bh, acc);
    acc = mfma16x16x32(ah, bl, acc);
    acc = mfma16x16x32(ah, bh, acc);
  }
}

// Store a value as a bf16 hi/lo pair (hi = rne(x), lo = rne(x - hi)).
__device__ __forceinline__ void st_split(__bf16* hi, __bf16* lo, int off, float x) {
  const __bf16 h = f32_to_bf16(x);
  hi[off] = h;
  lo[off] = f32_to_bf16(x - bf16_to_f32(h));
}

}  // namespace gdn2
