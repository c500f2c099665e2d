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
};

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
  float* dS_chunks;          // workspace [B,H,NC,Dk,Dv]: gradient of each chunk's exit state
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
  bool raw_gates = false;  // b, w, log_alpha hold pre-activations; db, dw, dlog_alpha are taken
                           // with respect to those
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
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
hipError_t launch_chain_bwd(const BwdArgs& a, const char* rec, hipStream_t stream);
hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream);
bool grad_supported(int Dk, int chunk, bool f32_inputs);

// Shapes with a compiled kernel (checked by the C ABI before launching).
bool fwd_supported(int Dk, int Dv, int chunk, bool f32_inputs);

}  // namespace gdn2
