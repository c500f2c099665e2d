// gdn2_api.hip -- the C ABI declared in include/gdn2.h: argument validation,
// workspace sizing, dispatch to the kernel launchers. No allocation, no host
// synchronisation, no state between calls.

#include <stdint.h>

#include <initializer_list>

#include "gdn2.h"
#include "gdn2_internal.h"

namespace {

constexpr int kVersion = 300;  // 0.3.0: the training pair (forward writes the backward records)
constexpr unsigned kKnownFlags =
    GDN2_FLAG_RAW_GATES | GDN2_FLAG_SCALAR_B | GDN2_FLAG_SCALAR_W | GDN2_FLAG_SCALAR_DECAY;

// the gate options of an argument block from the flags
template <class Args>
void set_gate_flags(Args& a, unsigned flags) {
  a.raw_gates = (flags & GDN2_FLAG_RAW_GATES) != 0;
  a.scalar_b = (flags & GDN2_FLAG_SCALAR_B) != 0;
  a.scalar_w = (flags & GDN2_FLAG_SCALAR_W) != 0;
  a.scalar_decay = (flags & GDN2_FLAG_SCALAR_DECAY) != 0;
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of sizes, dtype and pointer alignment. Returns GDN2_OK or an error.
int check_common(int B, int T, int H, int Dk, int Dv, int dt) {
  if (dt != GDN2_F32 && dt != GDN2_BF16) return GDN2_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return GDN2_ERR_SHAPE;
  // token indices are int32 inside the kernels
  if (T > (1 << 30)) return GDN2_ERR_SHAPE;
  if (!dim_ok(Dk) || !dim_ok(Dv)) return GDN2_ERR_UNSUPPORTED;
  return GDN2_OK;
}

int check_ptrs(std::initializer_list<const void*> required, std::initializer_list<const void*> optional) {
  for (const void* p : required)
    if (p == nullptr) return GDN2_ERR_NULL;
  for (const void* p : required)
    if (!aligned16(p)) return GDN2_ERR_ALIGN;
  for (const void* p : optional)
    if (p != nullptr && !aligned16(p)) return GDN2_ERR_ALIGN;
  return GDN2_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP; }

size_t state_bytes(int B, int H, int Dk, int Dv) { return (size_t)B * H * Dk * Dv * sizeof(float); }

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk, bool f32);

// The chunk that the backward and training-pair kernels tile a sequence with: the
// caller's, except where their LDS does not hold it (fp32 inputs at Dk = 128 with
// chunk 64), where they run 32-token chunks. The chunk size only tiles the
// recurrence: every size computes the same result up to rounding order.
int bwd_chunk(int Dk, int chunk, bool f32) {
  const auto fits = [&](int c) { return gdn2::grad_supported(Dk, c, f32) && gdn2::prep_fwd_supported(Dk, c, f32); };
  return (chunk == 64 && !fits(64) && fits(32)) ? 32 : chunk;
}

// The chunk of the single-pass forward (no workspace): likewise the caller's, or
// 32 where its LDS does not hold chunk 64.
int fwd_single_chunk(int Dk, int Dv, int chunk, bool f32) {
  return (chunk == 64 && !gdn2::fwd_supported(Dk, Dv, 64, f32) && gdn2::fwd_supported(Dk, Dv, 32, f32)) ? 32 : chunk;
}

// Backward plan: the two-stage reverse pass (chunk-parallel records, then the
// register-resident reverse chain), where the kernels cover the sizes (two_stage;
// otherwise the backward calls return GDN2_ERR_UNSUPPORTED), at the kernels'
// chunk (bwd_chunk).
struct BwdPlan {
  bool two_stage;
  int chunk;       // the kernels' chunk
  size_t part;     // one [B,H,NC,Dk,Dv] fp32 array, 256-byte aligned
  size_t records;  // records region (two-stage only): forward records for a
                   // state recompute, then the backward records
  size_t seg;      // the two-level reverse chain's segment maps (0: not used)
  size_t gsc;      // 16-bit inputs: partial maxima of the upstream gradients (grad_scale), 0 for fp32
  size_t need;
};

// the upstream-gradient partial maxima of nst (sequence, head) pairs (16-bit inputs only)
size_t gscale_bytes(int nst, bool f32) { return f32 ? 0 : al256((size_t)nst * gdn2::kGradScaleSplit * 4); }

BwdPlan bwd_plan(int B, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  BwdPlan p{};
  chunk = bwd_chunk(Dk, chunk, f32);
  p.chunk = chunk;
  const size_t nc = (size_t)((T + chunk - 1) / chunk);
  p.part = (nc * state_bytes(B, H, Dk, Dv) + 255) & ~(size_t)255;
  p.two_stage = gdn2::grad_supported(Dk, chunk, f32) && gdn2::prep_fwd_supported(Dk, chunk, f32);
  if (p.two_stage) {
    const size_t rb = (size_t)B * H * nc * gdn2::record_bytes(Dk, chunk, f32, 1);
    const size_t fw = fwd_workspace(B, T, H, Dk, Dv, chunk, f32);
    p.records = rb > fw ? rb : fw;
  }
  // gradient of every chunk's exit state, room to recompute the chunk entry
  // states when the caller passes none, the records, and the reverse chain's
  // segment maps for few heads and long sequences
  p.records = (p.records + 255) & ~(size_t)255;
  p.seg = al256(p.two_stage ? gdn2::fwd_seg_bytes(B, H, T, Dk, Dv, chunk) : 0);
  p.gsc = gscale_bytes(B * H, f32);
  p.need = 2 * p.part + p.records + p.seg + p.gsc;
  return p;
}


// The training pair's records buffer: the backward records, then (256-byte
// aligned) every chunk's entry state, fp32 for fp32 inputs and fp16 for 16-bit
// ones (the precision of their matrix-core uses in the backward); and the
// workspace of the backward that reads them (state gradients, then the reverse
// chain's segment maps).
size_t train_states_offset(int B, int T, int H, int Dk, int chunk, bool f32) {
  return al256((size_t)B * H * ((T + chunk - 1) / chunk) * gdn2::record_bytes(Dk, chunk, f32, 1));
}

size_t train_records(int B, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  return train_states_offset(B, T, H, Dk, chunk, f32) +
         (size_t)B * H * ((T + chunk - 1) / chunk) * Dk * Dv * (f32 ? 4 : 2);
}

// the training pair's backward workspace: state gradients, segment maps, upstream-gradient maxima
size_t bwd_records_workspace(const BwdPlan& p) { return p.part + p.seg + p.gsc; }

// Two-stage forward workspace: records, then T (w*v) for every chunk, then
// (256-byte aligned) the segment maps and entry states of the two-level chain
// when it is used for the sizes; 0 when the chunk-parallel kernel does not
// cover the sizes.
// T (w v) of one chunk: fp32 for fp32 inputs, fp16 for 16-bit ones
size_t ut_bytes(int chunk, int Dv, bool f32) { return (size_t)chunk * Dv * (f32 ? 4 : 2); }

size_t fwd_seg_offset(int B, int T, int H, int Dv, int Dk, int chunk, bool f32) {
  const size_t nchunks = (size_t)B * H * ((T + chunk - 1) / chunk);
  const size_t base = nchunks * (gdn2::fwd_record_bytes(Dk, chunk, f32) + ut_bytes(chunk, Dv, f32));
  return (base + 255) & ~(size_t)255;
}

size_t fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  if (!gdn2::prep_fwd_supported(Dk, chunk, f32)) return 0;
  const size_t nchunks = (size_t)B * H * ((T + chunk - 1) / chunk);
  const size_t base = nchunks * (gdn2::fwd_record_bytes(Dk, chunk, f32) + ut_bytes(chunk, Dv, f32));
  const size_t sb = gdn2::fwd_seg_bytes(B, H, T, Dk, Dv, chunk);
  return sb ? fwd_seg_offset(B, T, H, Dv, Dk, chunk, f32) + sb : base;
}

// the two-level chain's buffers inside a forward workspace (or records region), or null
char* fwd_seg_ptr(char* ws, int B, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  if (gdn2::fwd_seg_bytes(B, H, T, Dk, Dv, chunk) == 0) return nullptr;
  return ws + fwd_seg_offset(B, T, H, Dv, Dk, chunk, f32);
}

// Packed variable-length batches: [tables][...] workspaces. Forward: records
// and T (w v) over [H][max_chunks]; backward: state gradients and recomputed
// entry states ([H][max_chunks][Dk][Dv] each), then a records region for the
// forward records (state recompute) and the backward ones.
struct VarlenPlan {
  int L;             // segment length of the two-level chain (0: plain chain)
  size_t tables, part, records, seg_off, gsc_off, need;  // gsc_off: upstream-gradient maxima (backward)
};

VarlenPlan varlen_plan(int op, int N, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  VarlenPlan p{};
  const size_t mc = (size_t)gdn2::varlen_max_chunks(N, T, chunk);
  p.L = gdn2::varlen_seg_len(N, T, H, Dk, Dv, chunk);
  p.tables = al256(gdn2::varlen_table_bytes(N, T, chunk, p.L));
  // forward region: records, T (w v), then the two-level chain's segment maps
  p.seg_off = al256((size_t)H * mc * (gdn2::fwd_record_bytes(Dk, chunk, f32) + ut_bytes(chunk, Dv, f32)));
  const size_t fwd_rec = p.seg_off + gdn2::varlen_seg_bytes(N, T, H, Dk, Dv, chunk);
  if (op == GDN2_OP_FWD) {
    p.records = al256(fwd_rec);
    p.need = p.tables + p.records;
  } else if (op == GDN2_OP_BWD_RECORDS) {
    // the backward from the training pair's records: state gradients, then the
    // reverse chain's segment maps
    p.part = al256((size_t)H * mc * Dk * Dv * 4);
    p.gsc_off = p.tables + p.part + al256(gdn2::varlen_seg_bytes(N, T, H, Dk, Dv, chunk));
    p.need = p.gsc_off + gscale_bytes(N * H, f32);
  } else {
    p.part = al256((size_t)H * mc * Dk * Dv * 4);
    const size_t bwd_rec = (size_t)H * mc * gdn2::record_bytes(Dk, chunk, f32, 1);
    p.records = al256(bwd_rec > fwd_rec ? bwd_rec : fwd_rec);
    // then the reverse chain's segment maps, then the upstream-gradient maxima
    p.gsc_off = p.tables + 2 * p.part + p.records + al256(gdn2::varlen_seg_bytes(N, T, H, Dk, Dv, chunk));
    p.need = p.gsc_off + gscale_bytes(N * H, f32);
  }
  return p;
}

}  // namespace

namespace gdn2 {

// dst[i] = src ? src[i] : 0 -- a plain kernel rather than a memset/memcpy node so
// that the call can be captured into a HIP graph and replayed.
__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace gdn2

extern "C" {

int gdn2_version(void) { return kVersion; }

const char* gdn2_status_string(int status) {
  switch (status) {
    case GDN2_OK: return "GDN2_OK: success";
    case GDN2_ERR_NULL: return "GDN2_ERR_NULL: a required pointer is NULL";
    case GDN2_ERR_SHAPE: return "GDN2_ERR_SHAPE: a size is negative or too large";
    case GDN2_ERR_DTYPE: return "GDN2_ERR_DTYPE: unknown input dtype";
    case GDN2_ERR_ALIGN: return "GDN2_ERR_ALIGN: a pointer is not 16-byte aligned";
    case GDN2_ERR_UNSUPPORTED: return "GDN2_ERR_UNSUPPORTED: Dk, Dv or chunk not supported";
    case GDN2_ERR_WORKSPACE: return "GDN2_ERR_WORKSPACE: workspace missing or too small";
    case GDN2_ERR_HIP: return "GDN2_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "unknown gdn2 status";
}

size_t gdn2_workspace_bytes(int op, int B, int T, int H, int Dk, int Dv, int chunk, int dt) {
  if (check_common(B, T, H, Dk, Dv, dt) != GDN2_OK) return 0;
  if (op == GDN2_OP_BWD) {
    if (!chunk_ok(chunk) || T == 0) return 0;
    const BwdPlan p = bwd_plan(B, T, H, Dk, Dv, chunk, dt == GDN2_F32);
    return p.two_stage ? p.need : 0;
  }
  if (op == GDN2_OP_FWD) {
    if (!chunk_ok(chunk) || T == 0) return 0;
    // also enough for the training pair's forward, which runs at the backward's chunk
    const bool f32 = dt == GDN2_F32;
    const size_t own = fwd_workspace(B, T, H, Dk, Dv, chunk, f32);
    const int kc = bwd_chunk(Dk, chunk, f32);
    const size_t pair = kc != chunk && own ? fwd_workspace(B, T, H, Dk, Dv, kc, f32) : 0;
    return own > pair ? own : pair;
  }
  if (op == GDN2_OP_BWD_RECORDS) {
    if (!chunk_ok(chunk) || T == 0) return 0;
    const BwdPlan p = bwd_plan(B, T, H, Dk, Dv, chunk, dt == GDN2_F32);
    return p.two_stage ? bwd_records_workspace(p) : 0;
  }
  return 0;
}

size_t gdn2_records_bytes(int B, int T, int H, int Dk, int Dv, int chunk, int dt) {
  if (check_common(B, T, H, Dk, Dv, dt) != GDN2_OK || !chunk_ok(chunk) || T == 0) return 0;
  const bool f32 = dt == GDN2_F32;
  if (!bwd_plan(B, T, H, Dk, Dv, chunk, f32).two_stage) return 0;
  return train_records(B, T, H, Dk, Dv, bwd_chunk(Dk, chunk, f32), f32);
}

int gdn2_fwd_chunked_ex(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                        const void* w, const float* S0, float* o, float* S_final, float* chunk_states,
                        void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk, int Dv, int chunk,
                        int dt, unsigned flags, void* stream) {
  int st = check_common(B, T, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if ((flags & ~kKnownFlags) != 0) return GDN2_ERR_UNSUPPORTED;
  if (!chunk_ok(chunk)) return GDN2_ERR_UNSUPPORTED;
  // the two-stage path runs when a workspace is given and covers the sizes
  const bool two_stage = workspace != nullptr && gdn2::prep_fwd_supported(Dk, chunk, dt == GDN2_F32);
  const int kc1 = two_stage ? chunk : fwd_single_chunk(Dk, Dv, chunk, dt == GDN2_F32);
  if (!two_stage && !gdn2::fwd_supported(Dk, Dv, kc1, dt == GDN2_F32)) return GDN2_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    st = check_ptrs({}, {S0, S_final});
    if (st != GDN2_OK) return st;
    if (S_final == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(S_final, S0, (int64_t)B * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, o}, {S0, S_final, chunk_states});
  if (st != GDN2_OK) return st;
  gdn2::FwdArgs a{q, k, v, log_alpha, b, w, S0, o, S_final, chunk_states, B, T, H, Dk, Dv, chunk, dt == GDN2_F32};
  set_gate_flags(a, flags);
  if (!two_stage) {
    a.chunk = kc1;
    a.state_every = chunk / kc1;
    return hip_status(gdn2::launch_fwd(a, s));
  }
  const size_t need = fwd_workspace(B, T, H, Dk, Dv, chunk, dt == GDN2_F32);
  if (workspace_bytes < need) return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
  char* rec = static_cast<char*>(workspace);
  float* ut = reinterpret_cast<float*>(rec + (size_t)B * H * ((T + chunk - 1) / chunk) *
                                                 gdn2::fwd_record_bytes(Dk, chunk, dt == GDN2_F32));
  st = hip_status(gdn2::launch_prep_fwd(a, rec, ut, s));
  if (st != GDN2_OK) return st;
  return hip_status(
      gdn2::launch_chain_fwd(a, rec, ut, fwd_seg_ptr(rec, B, T, H, Dk, Dv, chunk, dt == GDN2_F32), s));
}

int gdn2_fwd_chunked(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                     const void* w, const float* S0, float* o, float* S_final, float* chunk_states,
                     void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk, int Dv, int chunk,
                     int dt, void* stream) {
  return gdn2_fwd_chunked_ex(q, k, v, log_alpha, b, w, S0, o, S_final, chunk_states, workspace, workspace_bytes, B,
                             T, H, Dk, Dv, chunk, dt, 0u, stream);
}

int gdn2_decode_step_ex(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                        const void* w, float* S, float* o, int B, int H, int Dk, int Dv, int dt, unsigned flags,
                        void* stream) {
  int st = check_common(B, 1, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if ((flags & ~kKnownFlags) != 0) return GDN2_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return GDN2_OK;
  st = check_ptrs({q, k, v, log_alpha, b, w, S, o}, {});
  if (st != GDN2_OK) return st;
  gdn2::DecodeArgs a{q, k, v, log_alpha, b, w, S, o, B, H, Dk, Dv, dt == GDN2_F32};
  set_gate_flags(a, flags);
  return hip_status(gdn2::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int gdn2_decode_step(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                     const void* w, float* S, float* o, int B, int H, int Dk, int Dv, int dt, void* stream) {
  return gdn2_decode_step_ex(q, k, v, log_alpha, b, w, S, o, B, H, Dk, Dv, dt, 0u, stream);
}

int gdn2_bwd_chunked_ex(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                        const void* w, const float* S0, const void* dO, const float* dS_final,
                        const float* chunk_states, float* dq, float* dk, float* dv, float* dlog_alpha, float* db,
                        float* dw, float* dS0, void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk,
                        int Dv, int chunk, int dt, unsigned flags, void* stream) {
  int st = check_common(B, T, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if ((flags & ~kKnownFlags) != 0) return GDN2_ERR_UNSUPPORTED;
  if (!chunk_ok(chunk)) return GDN2_ERR_UNSUPPORTED;
  const bool f32 = dt == GDN2_F32;
  const BwdPlan plan = bwd_plan(B, T, H, Dk, Dv, chunk, f32);
  if (!plan.two_stage) return GDN2_ERR_UNSUPPORTED;
  if (plan.chunk != chunk) {
    // the kernels run finer chunks: the caller's chunk states lack their entry
    // states, so they are recomputed
    chunk = plan.chunk;
    chunk_states = nullptr;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    // no tokens: S_T = S0, so dS0 = dS_final
    st = check_ptrs({}, {dS_final, dS0});
    if (st != GDN2_OK) return st;
    if (dS0 == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(dS0, dS_final, (int64_t)B * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, dO, dq, dk, dv, dlog_alpha, db, dw},
                  {S0, dS_final, chunk_states, dS0});
  if (st != GDN2_OK) return st;
  if (workspace == nullptr || workspace_bytes < plan.need) return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  float* dS_chunks = reinterpret_cast<float*>(ws);
  char* rec = ws + 2 * plan.part;
  float* states = const_cast<float*>(chunk_states);
  gdn2::FwdArgs f{q, k, v, log_alpha, b, w, S0, nullptr, nullptr, nullptr, B, T, H, Dk, Dv, chunk, f32};
  set_gate_flags(f, flags);
  if (states == nullptr) {
    states = reinterpret_cast<float*>(ws + plan.part);
    f.chunk_states = states;
    {
      // the two-stage forward (the default forward path, so the states match a
      // saved forward's bit for bit) in the records region; the backward
      // records overwrite it afterwards
      float* ut = reinterpret_cast<float*>(rec + (size_t)B * H * ((T + chunk - 1) / chunk) *
                                                     gdn2::fwd_record_bytes(Dk, chunk, f32));
      st = hip_status(gdn2::launch_prep_fwd(f, rec, ut, s));
      if (st == GDN2_OK)
        st = hip_status(gdn2::launch_chain_fwd(f, rec, ut, fwd_seg_ptr(rec, B, T, H, Dk, Dv, chunk, f32), s));
    }
    if (st != GDN2_OK) return st;
  }
  gdn2::BwdArgs a{q, k, v, log_alpha, b, w, dO, dS_final, states, dS_chunks, dq, dk, dv, dlog_alpha, db, dw,
                  dS0, B, T, H, Dk, Dv, chunk, f32};
  set_gate_flags(a, flags);
  if (!f32) {
    float* part = reinterpret_cast<float*>(ws + 2 * plan.part + plan.records + plan.seg);
    st = hip_status(gdn2::launch_grad_scale(a, part, s));
    a.gscale = part;
  }
  if (st == GDN2_OK) st = hip_status(gdn2::launch_prep_bwd(f, rec, s));
  if (st == GDN2_OK)
    st = hip_status(gdn2::launch_chain_bwd(a, rec, plan.seg ? rec + plan.records : nullptr, s));
  a.records = rec;
  if (st == GDN2_OK) st = hip_status(gdn2::launch_bwd_grad(a, s));
  return st;
}

int gdn2_fwd_chunked_train(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                           const void* w, const float* S0, float* o, float* S_final, void* records,
                           size_t records_bytes, void* workspace, size_t workspace_bytes, int B, int T, int H,
                           int Dk, int Dv, int chunk, int dt, unsigned flags, void* stream) {
  int st = check_common(B, T, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if ((flags & ~kKnownFlags) != 0 || !chunk_ok(chunk)) return GDN2_ERR_UNSUPPORTED;
  const bool f32 = dt == GDN2_F32;
  if (!bwd_plan(B, T, H, Dk, Dv, chunk, f32).two_stage) return GDN2_ERR_UNSUPPORTED;
  chunk = bwd_chunk(Dk, chunk, f32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0 || H == 0) return GDN2_OK;
  if (T == 0) {  // no chunks, no records: S_T = S0
    st = check_ptrs({}, {S0, S_final});
    if (st != GDN2_OK) return st;
    if (S_final == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(S_final, S0, (int64_t)B * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, o, records}, {S0, S_final});
  if (st != GDN2_OK) return st;
  const size_t need = fwd_workspace(B, T, H, Dk, Dv, chunk, f32);
  if (workspace == nullptr || workspace_bytes < need || records_bytes < train_records(B, T, H, Dk, Dv, chunk, f32))
    return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(records) & 255u) != 0)
    return GDN2_ERR_ALIGN;
  char* states = static_cast<char*>(records) + train_states_offset(B, T, H, Dk, chunk, f32);
  gdn2::FwdArgs a{q, k, v, log_alpha, b, w, S0, o, S_final, f32 ? reinterpret_cast<float*>(states) : nullptr,
                  B, T, H, Dk, Dv, chunk, f32};
  if (!f32) a.states16 = reinterpret_cast<_Float16*>(states);
  set_gate_flags(a, flags);
  char* rec = static_cast<char*>(workspace);
  float* ut = reinterpret_cast<float*>(rec + (size_t)B * H * ((T + chunk - 1) / chunk) *
                                                 gdn2::fwd_record_bytes(Dk, chunk, f32));
  st = hip_status(gdn2::launch_prep_train(a, rec, ut, static_cast<char*>(records), s));
  if (st != GDN2_OK) return st;
  return hip_status(gdn2::launch_chain_fwd(a, rec, ut, fwd_seg_ptr(rec, B, T, H, Dk, Dv, chunk, f32), s));
}

int gdn2_bwd_chunked_records(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                             const void* w, const void* dO, const float* dS_final, const void* records,
                             size_t records_bytes, float* dq, float* dk, float* dv, float* dlog_alpha, float* db,
                             float* dw, float* dS0, void* workspace, size_t workspace_bytes, int B, int T, int H,
                             int Dk, int Dv, int chunk, int dt, unsigned flags, void* stream) {
  int st = check_common(B, T, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if ((flags & ~kKnownFlags) != 0 || !chunk_ok(chunk)) return GDN2_ERR_UNSUPPORTED;
  const bool f32 = dt == GDN2_F32;
  const BwdPlan plan = bwd_plan(B, T, H, Dk, Dv, chunk, f32);
  if (!plan.two_stage) return GDN2_ERR_UNSUPPORTED;
  chunk = plan.chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0 || H == 0) return GDN2_OK;
  if (T == 0) {  // S_T = S0, so dS0 = dS_final
    st = check_ptrs({}, {dS_final, dS0});
    if (st != GDN2_OK) return st;
    if (dS0 == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(dS0, dS_final, (int64_t)B * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, dO, records, dq, dk, dv, dlog_alpha, db, dw}, {dS_final, dS0});
  if (st != GDN2_OK) return st;
  if (workspace == nullptr || workspace_bytes < bwd_records_workspace(plan) ||
      records_bytes < train_records(B, T, H, Dk, Dv, chunk, f32))
    return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(records) & 255u) != 0)
    return GDN2_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  const char* rec = static_cast<const char*>(records);
  const char* states = rec + train_states_offset(B, T, H, Dk, chunk, f32);
  gdn2::BwdArgs a{q,  k,  v,  log_alpha,  b,  w,  dO, dS_final, f32 ? reinterpret_cast<const float*>(states) : nullptr,
                  reinterpret_cast<float*>(ws), dq, dk, dv, dlog_alpha, db, dw, dS0, B, T, H, Dk, Dv, chunk, f32};
  if (!f32) a.states16 = reinterpret_cast<const _Float16*>(states);
  set_gate_flags(a, flags);
  if (!f32) {
    float* part = reinterpret_cast<float*>(ws + plan.part + plan.seg);
    st = hip_status(gdn2::launch_grad_scale(a, part, s));
    a.gscale = part;
  }
  if (st == GDN2_OK) st = hip_status(gdn2::launch_chain_bwd(a, rec, plan.seg ? ws + plan.part : nullptr, s));
  a.records = rec;
  if (st == GDN2_OK) st = hip_status(gdn2::launch_bwd_grad(a, s));
  return st;
}

int gdn2_bwd_chunked(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                     const void* w, const float* S0, const void* dO, const float* dS_final,
                     const float* chunk_states, float* dq, float* dk, float* dv, float* dlog_alpha, float* db,
                     float* dw, float* dS0, void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk,
                     int Dv, int chunk, int dt, void* stream) {
  return gdn2_bwd_chunked_ex(q, k, v, log_alpha, b, w, S0, dO, dS_final, chunk_states, dq, dk, dv, dlog_alpha, db,
                             dw, dS0, workspace, workspace_bytes, B, T, H, Dk, Dv, chunk, dt, 0u, stream);
}

// ---- packed variable-length batches ----

int gdn2_varlen_max_chunks(int N, int T, int chunk) {
  if (N < 0 || T < 0 || !chunk_ok(chunk)) return -1;
  return gdn2::varlen_max_chunks(N, T, chunk);
}

size_t gdn2_varlen_workspace_bytes(int op, int N, int T, int H, int Dk, int Dv, int chunk, int dt) {
  if (check_common(1, T, H, Dk, Dv, dt) != GDN2_OK || N < 0 || !chunk_ok(chunk)) return 0;
  if (op != GDN2_OP_FWD && op != GDN2_OP_BWD && op != GDN2_OP_BWD_RECORDS) return 0;
  const bool f32 = dt == GDN2_F32;
  if (!gdn2::prep_fwd_supported(Dk, chunk, f32)) return 0;
  const int kc = bwd_chunk(Dk, chunk, f32);
  if (op != GDN2_OP_FWD)
    return gdn2::grad_supported(Dk, kc, f32) ? varlen_plan(op, N, T, H, Dk, Dv, kc, f32).need : 0;
  // also enough for the training pair's forward, which runs at the backward's chunk
  const size_t own = varlen_plan(op, N, T, H, Dk, Dv, chunk, f32).need;
  const size_t pair = kc != chunk && gdn2::prep_fwd_supported(Dk, kc, f32)
                          ? varlen_plan(op, N, T, H, Dk, Dv, kc, f32).need : 0;
  return own > pair ? own : pair;
}

// The packed-batch training pair's records buffer: backward records over
// [H][max_chunks], then (256-byte aligned) the chunk entry states over
// [H][max_chunks] (fp16 for 16-bit inputs), as for the dense pair.
static size_t varlen_train_states_offset(int N, int T, int H, int Dk, int chunk, bool f32) {
  return al256((size_t)H * gdn2::varlen_max_chunks(N, T, chunk) * gdn2::record_bytes(Dk, chunk, f32, 1));
}

static size_t varlen_train_records(int N, int T, int H, int Dk, int Dv, int chunk, bool f32) {
  return varlen_train_states_offset(N, T, H, Dk, chunk, f32) +
         (size_t)H * gdn2::varlen_max_chunks(N, T, chunk) * Dk * Dv * (f32 ? 4 : 2);
}

size_t gdn2_varlen_records_bytes(int N, int T, int H, int Dk, int Dv, int chunk, int dt) {
  if (gdn2_varlen_workspace_bytes(GDN2_OP_BWD_RECORDS, N, T, H, Dk, Dv, chunk, dt) == 0) return 0;
  return varlen_train_records(N, T, H, Dk, Dv, bwd_chunk(Dk, chunk, dt == GDN2_F32), dt == GDN2_F32);
}

static int varlen_common(const int64_t* cu_seqlens, int N, int T, int H, int Dk, int Dv, int chunk, int dt,
                         unsigned flags, int op) {
  int st = check_common(1, T, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if (N < 0 || T > (1 << 30) - N * 64) return GDN2_ERR_SHAPE;
  if ((flags & ~kKnownFlags) != 0 || !chunk_ok(chunk)) return GDN2_ERR_UNSUPPORTED;
  const bool f32 = dt == GDN2_F32;
  if (!gdn2::prep_fwd_supported(Dk, chunk, f32) || (op == GDN2_OP_BWD && !gdn2::grad_supported(Dk, chunk, f32)))
    return GDN2_ERR_UNSUPPORTED;
  if (N > 0 && cu_seqlens == nullptr) return GDN2_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0) return GDN2_ERR_ALIGN;
  return GDN2_OK;
}

int gdn2_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                    const void* w, const long long* cu_seqlens_, int N, const float* S0, float* o, float* S_final,
                    float* chunk_states, void* workspace, size_t workspace_bytes, int T, int H, int Dk, int Dv,
                    int chunk, int dt, unsigned flags, void* stream) {
  const int64_t* cu_seqlens = reinterpret_cast<const int64_t*>(cu_seqlens_);
  int st = varlen_common(cu_seqlens, N, T, H, Dk, Dv, chunk, dt, flags, GDN2_OP_FWD);
  if (st != GDN2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    st = check_ptrs({}, {S0, S_final});
    if (st != GDN2_OK) return st;
    if (S_final == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(S_final, S0, (int64_t)N * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, o}, {S0, S_final, chunk_states});
  if (st != GDN2_OK) return st;
  const bool f32 = dt == GDN2_F32;
  const VarlenPlan p = varlen_plan(GDN2_OP_FWD, N, T, H, Dk, Dv, chunk, f32);
  if (workspace == nullptr || workspace_bytes < p.need) return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  gdn2::FwdArgs a{q, k, v, log_alpha, b, w, S0, o, S_final, chunk_states, 1, T, H, Dk, Dv, chunk, f32};
  set_gate_flags(a, flags);
  st = hip_status(gdn2::launch_varlen_plan(cu_seqlens, N, T, chunk, p.L, ws, a.vl, s));
  if (st != GDN2_OK) return st;
  char* rec = ws + p.tables;
  float* ut = reinterpret_cast<float*>(rec + (size_t)H * a.vl.max_chunks * gdn2::fwd_record_bytes(Dk, chunk, f32));
  st = hip_status(gdn2::launch_prep_fwd(a, rec, ut, s));
  if (st != GDN2_OK) return st;
  return hip_status(gdn2::launch_chain_fwd(a, rec, ut, p.L > 0 ? rec + p.seg_off : nullptr, s));
}

int gdn2_bwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                    const void* w, const long long* cu_seqlens_, int N, const float* S0, const void* dO,
                    const float* dS_final, const float* chunk_states, float* dq, float* dk, float* dv,
                    float* dlog_alpha, float* db, float* dw, float* dS0, void* workspace, size_t workspace_bytes,
                    int T, int H, int Dk, int Dv, int chunk, int dt, unsigned flags, void* stream) {
  const int64_t* cu_seqlens = reinterpret_cast<const int64_t*>(cu_seqlens_);
  const int caller_chunk = chunk;
  chunk = bwd_chunk(Dk, chunk, dt == GDN2_F32);
  int st = varlen_common(cu_seqlens, N, T, H, Dk, Dv, chunk, dt, flags, GDN2_OP_BWD);
  if (st != GDN2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    st = check_ptrs({}, {dS_final, dS0});
    if (st != GDN2_OK) return st;
    if (dS0 == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(dS0, dS_final, (int64_t)N * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, dO, dq, dk, dv, dlog_alpha, db, dw}, {S0, dS_final, chunk_states, dS0});
  if (st != GDN2_OK) return st;
  const bool f32 = dt == GDN2_F32;
  const VarlenPlan p = varlen_plan(GDN2_OP_BWD, N, T, H, Dk, Dv, chunk, f32);
  if (workspace == nullptr || workspace_bytes < p.need) return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  gdn2::FwdArgs f{q, k, v, log_alpha, b, w, S0, nullptr, nullptr, nullptr, 1, T, H, Dk, Dv, chunk, f32};
  set_gate_flags(f, flags);
  st = hip_status(gdn2::launch_varlen_plan(cu_seqlens, N, T, chunk, p.L, ws, f.vl, s));
  if (st != GDN2_OK) return st;
  float* dS_chunks = reinterpret_cast<float*>(ws + p.tables);
  char* rec = ws + p.tables + 2 * p.part;
  // finer kernel chunks than the caller's: its chunk states lack their entry states, so they are recomputed
  float* states = caller_chunk == chunk ? const_cast<float*>(chunk_states) : nullptr;
  if (states == nullptr) {
    // the entry states from the two-stage forward, in the records region first
    states = reinterpret_cast<float*>(ws + p.tables + p.part);
    f.chunk_states = states;
    float* ut = reinterpret_cast<float*>(rec + (size_t)H * f.vl.max_chunks * gdn2::fwd_record_bytes(Dk, chunk, f32));
    st = hip_status(gdn2::launch_prep_fwd(f, rec, ut, s));
    if (st == GDN2_OK)
      st = hip_status(gdn2::launch_chain_fwd(f, rec, ut, p.L > 0 ? rec + p.seg_off : nullptr, s));
    if (st != GDN2_OK) return st;
  }
  gdn2::BwdArgs a{q, k, v, log_alpha, b, w, dO, dS_final, states, dS_chunks, dq, dk, dv, dlog_alpha, db, dw,
                  dS0, 1, T, H, Dk, Dv, chunk, f32};
  set_gate_flags(a, flags);
  a.vl = f.vl;
  if (!f32) {
    float* part = reinterpret_cast<float*>(ws + p.gsc_off);
    st = hip_status(gdn2::launch_grad_scale(a, part, s));
    a.gscale = part;
  }
  if (st == GDN2_OK) st = hip_status(gdn2::launch_prep_bwd(f, rec, s));
  if (st == GDN2_OK) st = hip_status(gdn2::launch_chain_bwd(a, rec, p.L > 0 ? rec + p.records : nullptr, s));
  a.records = rec;
  if (st == GDN2_OK) st = hip_status(gdn2::launch_bwd_grad(a, s));
  return st;
}

int gdn2_fwd_varlen_train(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                          const void* w, const long long* cu_seqlens_, int N, const float* S0, float* o,
                          float* S_final, void* records, size_t records_bytes, void* workspace,
                          size_t workspace_bytes, int T, int H, int Dk, int Dv, int chunk, int dt, unsigned flags,
                          void* stream) {
  const int64_t* cu_seqlens = reinterpret_cast<const int64_t*>(cu_seqlens_);
  chunk = bwd_chunk(Dk, chunk, dt == GDN2_F32);
  int st = varlen_common(cu_seqlens, N, T, H, Dk, Dv, chunk, dt, flags, GDN2_OP_BWD);
  if (st != GDN2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    st = check_ptrs({}, {S0, S_final});
    if (st != GDN2_OK) return st;
    if (S_final == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(S_final, S0, (int64_t)N * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, o, records}, {S0, S_final});
  if (st != GDN2_OK) return st;
  const bool f32 = dt == GDN2_F32;
  const VarlenPlan p = varlen_plan(GDN2_OP_FWD, N, T, H, Dk, Dv, chunk, f32);
  if (workspace == nullptr || workspace_bytes < p.need ||
      records_bytes < varlen_train_records(N, T, H, Dk, Dv, chunk, f32))
    return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(records) & 255u) != 0)
    return GDN2_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  char* states = static_cast<char*>(records) + varlen_train_states_offset(N, T, H, Dk, chunk, f32);
  gdn2::FwdArgs a{q, k, v, log_alpha, b, w, S0, o, S_final, f32 ? reinterpret_cast<float*>(states) : nullptr,
                  1, T, H, Dk, Dv, chunk, f32};
  if (!f32) a.states16 = reinterpret_cast<_Float16*>(states);
  set_gate_flags(a, flags);
  st = hip_status(gdn2::launch_varlen_plan(cu_seqlens, N, T, chunk, p.L, ws, a.vl, s));
  if (st != GDN2_OK) return st;
  char* rec = ws + p.tables;
  float* ut = reinterpret_cast<float*>(rec + (size_t)H * a.vl.max_chunks * gdn2::fwd_record_bytes(Dk, chunk, f32));
  st = hip_status(gdn2::launch_prep_train(a, rec, ut, static_cast<char*>(records), s));
  if (st != GDN2_OK) return st;
  return hip_status(gdn2::launch_chain_fwd(a, rec, ut, p.L > 0 ? rec + p.seg_off : nullptr, s));
}

int gdn2_bwd_varlen_records(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                            const void* w, const long long* cu_seqlens_, int N, const void* dO,
                            const float* dS_final, const void* records, size_t records_bytes, float* dq, float* dk,
                            float* dv, float* dlog_alpha, float* db, float* dw, float* dS0, void* workspace,
                            size_t workspace_bytes, int T, int H, int Dk, int Dv, int chunk, int dt,
                            unsigned flags, void* stream) {
  const int64_t* cu_seqlens = reinterpret_cast<const int64_t*>(cu_seqlens_);
  chunk = bwd_chunk(Dk, chunk, dt == GDN2_F32);
  int st = varlen_common(cu_seqlens, N, T, H, Dk, Dv, chunk, dt, flags, GDN2_OP_BWD);
  if (st != GDN2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0 || H == 0) return GDN2_OK;
  if (T == 0) {
    st = check_ptrs({}, {dS_final, dS0});
    if (st != GDN2_OK) return st;
    if (dS0 == nullptr) return GDN2_OK;
    return hip_status(gdn2::launch_copy_or_zero(dS0, dS_final, (int64_t)N * H * Dk * Dv, s));
  }
  st = check_ptrs({q, k, v, log_alpha, b, w, dO, records, dq, dk, dv, dlog_alpha, db, dw}, {dS_final, dS0});
  if (st != GDN2_OK) return st;
  const bool f32 = dt == GDN2_F32;
  const VarlenPlan p = varlen_plan(GDN2_OP_BWD_RECORDS, N, T, H, Dk, Dv, chunk, f32);
  if (workspace == nullptr || workspace_bytes < p.need ||
      records_bytes < varlen_train_records(N, T, H, Dk, Dv, chunk, f32))
    return GDN2_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (reinterpret_cast<uintptr_t>(records) & 255u) != 0)
    return GDN2_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  const char* rec = static_cast<const char*>(records);
  const char* states = rec + varlen_train_states_offset(N, T, H, Dk, chunk, f32);
  gdn2::BwdArgs a{q,  k,  v,  log_alpha,  b,  w,  dO, dS_final, f32 ? reinterpret_cast<const float*>(states) : nullptr,
                  reinterpret_cast<float*>(ws + p.tables), dq, dk, dv, dlog_alpha, db, dw, dS0, 1, T, H, Dk, Dv,
                  chunk, f32};
  if (!f32) a.states16 = reinterpret_cast<const _Float16*>(states);
  set_gate_flags(a, flags);
  st = hip_status(gdn2::launch_varlen_plan(cu_seqlens, N, T, chunk, p.L, ws, a.vl, s));
  if (st == GDN2_OK && !f32) {
    float* part = reinterpret_cast<float*>(ws + p.gsc_off);
    st = hip_status(gdn2::launch_grad_scale(a, part, s));
    a.gscale = part;
  }
  if (st == GDN2_OK) st = hip_status(gdn2::launch_chain_bwd(a, rec, p.L > 0 ? ws + p.tables + p.part : nullptr, s));
  a.records = rec;
  if (st == GDN2_OK) st = hip_status(gdn2::launch_bwd_grad(a, s));
  return st;
}

int gdn2_decode_step_slots(const void* q, const void* k, const void* v, const float* log_alpha, const void* b,
                           const void* w, float* S_pool, const int* slots, int num_slots, float* o, int B, int H,
                           int Dk, int Dv, int dt, unsigned flags, void* stream) {
  int st = check_common(B, 1, H, Dk, Dv, dt);
  if (st != GDN2_OK) return st;
  if (num_slots < 0) return GDN2_ERR_SHAPE;
  if ((flags & ~kKnownFlags) != 0) return GDN2_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return GDN2_OK;
  st = check_ptrs({q, k, v, log_alpha, b, w, o}, {S_pool});
  if (st != GDN2_OK) return st;
  if (slots == nullptr || (num_slots > 0 && S_pool == nullptr)) return GDN2_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(slots) & 3u) != 0) return GDN2_ERR_ALIGN;
  gdn2::DecodeArgs a{q, k, v, log_alpha, b, w, S_pool, o, B, H, Dk, Dv, dt == GDN2_F32};
  set_gate_flags(a, flags);
  a.slots = slots;
  a.num_slots = num_slots;
  return hip_status(gdn2::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
