// gdn2_internal.h -- argument blocks and launchers shared between the C ABI
// (gdn2_api.hip) and the kernel translation units. Not a public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const void* b;
  const void* w;
  float* S;
  float* o;
  int B, H, Dk, Dv;
  bool f32_inputs;
  bool raw_gates = false;  // b, w, log_alpha hold pre-activations (sigmoid, sigmoid, -softplus)
  const int* slots = nullptr;  // [B]: state pool slot of each entry (S is then [num_slots, H, Dk, Dv])
  int num_slots = 0;
  bool scalar_b = false, scalar_w = false, scalar_decay = false;  // one value per (entry, head): [B, H]
};

// Variable-length packed batch: N sequences packed along T of a [1, T, H, D]
// layout. Chunks never cross a sequence boundary; chunk-indexed arrays
// (records, chunk states, state gradients) are [H][max_chunks] with the
// sequences' chunks in order, max_chunks = T / chunk + N bounding their count.
struct Varlen {
  const int64_t* cu = nullptr;       // [N+1] offsets, clamped non-decreasing within [0, T]; null: dense
  const int* chunk_seq = nullptr;    // [max_chunks] sequence of global chunk g, -1 past the last chunk
  const int* chunk_first = nullptr;  // [N+1] first global chunk of each sequence (prefix sums)
  int nseq = 0;
  int max_chunks = 0;
  // two-level chain inside the sequences (seg_len > 0): each sequence's chunks cut
  // into segments of seg_len chunks; segment-indexed arrays are [H][max_segs]
  const int* seg_first = nullptr;    // [N+1] first global segment of each sequence
  const int* seg_seq = nullptr;      // [max_segs] sequence of global segment s, -1 past the last
  int seg_len = 0;
  int max_segs = 0;
};

// Location of one chunk of a chunk-parallel grid. Dense: item = (b*H + h) * NC + n
// (chunk fastest). Varlen: item = h * max_chunks + g (g the global chunk).
struct ChunkLoc {
  int64_t item;   // index into the chunk-indexed arrays
  int64_t state;  // (batch row or sequence) * H + head: index of its states [., H, Dk, Dv]
  int64_t baseK;  // element offset of token 0 of the chunk's (batch row, head) in [., T, H, Dk]
  int64_t baseV;  // same in [., T, H, Dv]
  int t0;         // first token of the chunk (added to base* as (t0 + r) * H * D)
  int Lr;         // valid rows, 0 < Lr <= C; 0: no chunk (varlen grid past the last chunk)
};

__device__ __forceinline__ ChunkLoc chunk_loc(const Varlen& vl, int T, int H, int Dk, int Dv, int C, int NC,
                                              int item) {
  ChunkLoc L;
  L.item = item;
  if (vl.cu == nullptr) {
    const int bh = item / NC, n = item - bh * NC, bi = bh / H, h = bh - bi * H;
    L.state = bh;
    L.baseK = ((int64_t)bi * T * H + h) * Dk;
    L.baseV = ((int64_t)bi * T * H + h) * Dv;
    L.t0 = n * C;
    L.Lr = min(C, T - L.t0);
  } else {
    const int h = item / vl.max_chunks, g = item - h * vl.max_chunks;
    const int sq = vl.chunk_seq[g];
    L.state = (int64_t)(sq < 0 ? 0 : sq) * H + h;
    L.baseK = (int64_t)h * Dk;
    L.baseV = (int64_t)h * Dv;
    if (sq < 0) {
      L.t0 = 0;
      L.Lr = 0;
    } else {
      const int nl = g - vl.chunk_first[sq];
      const int64_t s0 = vl.cu[sq], len = vl.cu[sq + 1] - s0;
      L.t0 = (int)(s0 + (int64_t)nl * C);
      const int64_t rest = len - (int64_t)nl * C;
      L.Lr = (int)(rest < C ? rest : C);
    }
  }
  return L;
}

// Workgroups of a chunk-parallel grid (one per chunk location) and of a chain
// grid (one per (sequence or batch row, head)).
__host__ __device__ inline int64_t chunk_items(const Varlen& vl, int B, int T, int H, int C) {
  return vl.cu ? (int64_t)H * vl.max_chunks : (int64_t)B * H * ((T + C - 1) / C);
}
__host__ __device__ inline int seq_items(const Varlen& vl, int B, int H) { return (vl.cu ? vl.nseq : B) * H; }

// The item (chunk_loc's index) that workgroup blk of a chunk-parallel pass takes: head fastest, so that the
// workgroups in flight together read whole token rows of q, k, v, ... ([., T, H, D]: all heads of a token
// are adjacent) instead of one head's slice of many rows.
__device__ __forceinline__ int chunk_item_of_block(const Varlen& vl, int T, int H, int C, int blk) {
  if (vl.cu == nullptr) {
    const int NC = (T + C - 1) / C;
    const int bi = blk / (NC * H), rem = blk - bi * (NC * H), n = rem / H, h = rem - n * H;
    return (bi * H + h) * NC + n;
  }
  const int g = blk / H, h = blk - g * H;
  return h * vl.max_chunks + g;
}

// Location of one (sequence, head) walked by a chain kernel: its chunks are
// item0 .. item0 + nchunks - 1 in the chunk-indexed arrays, chunk n covers
// tokens tok0 + n*C .. of length min(C, len - n*C); state index for S0/S_final.
struct SeqLoc {
  int64_t item0, state, baseK, baseV;
  int tok0, len, nchunks;
};

// sb = b*H + h (dense) or seq*H + h (varlen)
__device__ __forceinline__ SeqLoc seq_loc(const Varlen& vl, int T, int H, int Dk, int Dv, int C, int sb) {
  SeqLoc S;
  S.state = sb;
  const int sq = sb / H, h = sb - sq * H;
  if (vl.cu == nullptr) {
    const int NC = (T + C - 1) / C;
    S.item0 = (int64_t)sb * NC;
    S.baseK = ((int64_t)sq * T * H + h) * Dk;
    S.baseV = ((int64_t)sq * T * H + h) * Dv;
    S.tok0 = 0;
    S.len = T;
    S.nchunks = NC;
  } else {
    S.item0 = (int64_t)h * vl.max_chunks + vl.chunk_first[sq];
    S.baseK = (int64_t)h * Dk;
    S.baseV = (int64_t)h * Dv;
    S.tok0 = (int)vl.cu[sq];
    S.len = (int)(vl.cu[sq + 1] - vl.cu[sq]);
    S.nchunks = vl.chunk_first[sq + 1] - vl.chunk_first[sq];
  }
  return S;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const void* b;
  const void* w;
  const float* S0;       // nullable
  float* o;
  float* S_final;        // nullable
  float* chunk_states;   // nullable
  int B, T, H, Dk, Dv, chunk;
  bool f32_inputs;
  bool raw_gates = false;  // b, w, log_alpha hold pre-activations (sigmoid, sigmoid, -softplus)
  _Float16* states16 = nullptr;  // two-stage chain only: the chunk entry states in fp16 (instead of
                                 // chunk_states), for the training pair's backward
  Varlen vl;               // packed variable-length batch (B = 1), or dense
  // gates of one value per (token, head), [., T, H], broadcast over their channels
  bool scalar_b = false, scalar_w = false, scalar_decay = false;
  int state_every = 1;     // single-pass forward: chunk_states holds the entry state of every
                           // state_every-th chunk (the kernel's chunk is 1/state_every of the caller's)
};

// Segmented (two-level) forward chain: the pass and its buffers.
constexpr int kSegMap = 1;  // zero-entry segments -> M (identity columns) and N (value columns)
constexpr int kSegRun = 2;  // segments from their true entry states -> o, chunk states, S_final
struct SegArgs {
  int nseg = 0;             // segments per (batch, head)
  int seg_len = 0;          // chunks per segment (the last one may be shorter)
  int mode = 0;
  float* M = nullptr;       // [B*H][nseg][Dk][Dk]
  float* N = nullptr;       // [B*H][nseg][Dk][Dv]
  float* S_in = nullptr;    // [B*H][nseg][Dk][Dv]: entry state of segment s (s >= 1)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const void* b;
  const void* w;
  const void* dO;
  const float* dS_final;     // nullable
  const float* chunk_states; // required here (the C ABI fills it in when the caller passes none)
  void* dS_chunks;           // workspace [B,H,NC,Dk,Dv]: gradient of each chunk's exit state, fp32 for
                             // fp32 inputs, fp16 for bf16 inputs (the precision of its matrix-core uses)
  float* dq;
  float* dk;
  float* dv;
  float* dlog_alpha;
  float* db;
  float* dw;
  float* dS0;                // nullable
  int B, T, H, Dk, Dv, chunk;
  bool f32_inputs;
  const char* records = nullptr;  // backward records (T, P^T, Kh, Kb) for launch_bwd_grad
  const _Float16* states16 = nullptr;  // the chunk entry states in fp16 (16-bit inputs): read instead of
                                       // chunk_states by launch_bwd_grad
  bool raw_gates = false;  // b, w, log_alpha hold pre-activations; db, dw, dlog_alpha are taken
                           // with respect to those
  Varlen vl;               // packed variable-length batch (B = 1), or dense
  // gates of one value per (token, head), [., T, H]; their gradients are then [., T, H] too
  // (summed over the channels the value is broadcast to)
  bool scalar_b = false, scalar_w = false, scalar_decay = false;
  // 16-bit inputs: partial maxima of |dO| and |dS_final| per (sequence, head), kGradScaleSplit each
  // (gdn2_grad_scale_kernel); the backward kernels scale dO and dS_final by grad_scale() of them
  const float* gscale = nullptr;
};

// Upstream-gradient scaling of the 16-bit backward. The backward is linear in (dO, dS_final) jointly,
// and their matrix-core operands are fp16 (range 6.1e-5 .. 65504 for normal numbers, while bf16 inputs
// span fp32's range): every (sequence, head) runs on dO and dS_final times a power of two that brings
// their largest magnitude into [1, 2), and every gradient is multiplied back on its store (exact).
constexpr int kGradScaleSplit = 8;  // partial maxima per (sequence, head)
__device__ __forceinline__ float grad_scale(const float* part, int64_t st) {
  if (part == nullptr) return 1.f;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kGradScaleSplit; ++i) m = fmaxf(m, part[st * kGradScaleSplit + i]);
  if (!(m > 0.f) || !(m <= 3.4e38f)) return 1.f;  // all zero, or not finite: unscaled
  int e = ilogbf(m);
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  return ldexpf(1.f, -e);
}
hipError_t launch_grad_scale(const BwdArgs& a, float* part, hipStream_t s);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Packed variable-length batches: table bytes in a workspace, the bound on the
// number of chunks, and the device-side plan that fills the tables and vl.
int varlen_max_chunks(int N, int T, int C);
// segment length of the two-level chain for a packed batch (0: plain chain), the
// bound on the number of segments, and the bytes of the segment maps
int varlen_seg_len(int N, int T, int H, int Dk, int Dv, int C);
int varlen_max_segs(int N, int T, int C, int L);
size_t varlen_seg_bytes(int N, int T, int H, int Dk, int Dv, int C);
size_t varlen_table_bytes(int N, int T, int C, int L);
hipError_t launch_varlen_plan(const int64_t* cu, int N, int T, int C, int L, char* tables, Varlen& vl,
                              hipStream_t s);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Two-stage forward: chunk-parallel records, then the sequential chain.
// rec: B*H*NC records of fwd_record_bytes(); ut: B*H*NC*C*Dv floats.
hipError_t launch_prep_fwd(const FwdArgs& a, char* rec, float* ut, hipStream_t stream);
// seg: nullable buffer of fwd_seg_bytes() bytes; used (two-level chain) when
// fwd_segments() > 1 for the sizes.
hipError_t launch_chain_fwd(const FwdArgs& a, const char* rec, const float* ut, char* seg, hipStream_t stream);
int fwd_segments(int B, int H, int T, int Dk, int Dv, int chunk);
size_t fwd_seg_bytes(int B, int H, int T, int Dk, int Dv, int chunk);
bool prep_fwd_supported(int Dk, int chunk, bool f32_inputs);
size_t fwd_record_bytes(int Dk, int chunk, bool f32_inputs);
// dir 0: forward record, 1: backward record (gdn2_frag.h)
size_t record_bytes(int Dk, int chunk, bool f32_inputs, int dir);

// Two-stage reverse pass of the backward: chunk-parallel backward records
// (B*H*NC of record_bytes(.., 1)), then the reverse state-gradient chain,
// which writes a.dS_chunks and a.dS0; launch_bwd_grad then forms the
// per-token gradients.
hipError_t launch_prep_bwd(const FwdArgs& a, char* rec, hipStream_t stream);
// Training forward's record pass: the forward records and T (w v) as
// launch_prep_fwd, and in the same pass the backward records into brec (as
// launch_prep_bwd would write them).
hipError_t launch_prep_train(const FwdArgs& a, char* rec, float* ut, char* brec, hipStream_t stream);
// seg: nullable buffer of fwd_seg_bytes() (dense) or varlen_seg_bytes() (packed)
// bytes; used (two-level reverse chain) under the same conditions as the forward's.
hipError_t launch_chain_bwd(const BwdArgs& a, const char* rec, char* seg, hipStream_t stream);
hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream);
bool grad_supported(int Dk, int chunk, bool f32_inputs);

// Shapes with a compiled kernel (checked by the C ABI before launching).
bool fwd_supported(int Dk, int Dv, int chunk, bool f32_inputs);

}  // namespace gdn2
