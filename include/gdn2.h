/*
 * gdn2.h -- C ABI of the Gated Delta Rule-2 (GDN-2) operator on AMD Instinct
 * MI355X (gfx950).
 *
 * The operator (per batch row b and head h; S_t is a Dk x Dv matrix):
 *
 *     S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t,          alpha_t = exp(log_alpha_t)
 *
 * with b_t in [0,1]^Dk the channel-wise erase gate (key side), w_t in
 * [0,1]^Dv the channel-wise write gate (value side) and alpha_t the
 * channel-wise decay on the key axis. Sources: the NVlabs/GatedDeltaNet-2
 * README ("Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"),
 * its gate bullet list and the update-rule paragraph after it (the page text
 * lacks the equation; the paragraph puts the erase gate on the key side of the
 * rank-one erase and the write gate on the value side of the write), and the
 * arXiv 2605.22791 abstract (the update as a fast-weight write, the delta
 * rule, the reductions to KDA and Gated DeltaNet, the chunkwise WY algorithm,
 * the gate-aware backward, decoding in constant memory).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a device pointer owned by the caller. The library
 *   allocates nothing, keeps no state between calls and is thread-safe.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL is the default stream). No host synchronisation happens inside.
 * - Tensors are contiguous, row-major, with 16-byte-aligned base pointers.
 *     q, k, b, log_alpha and their gradients : [B, T, H, Dk]
 *     v, w, dO, o and their gradients        : [B, T, H, Dv]
 *     states S0, S_final, dS_final, dS0      : [B, H, Dk, Dv]  fp32
 *     chunk_states                           : [B, H, NC, Dk, Dv] fp32,
 *       NC = ceil(T / chunk); entry n is the state entering chunk n
 *       (entry 0 is S0).
 *     Decode drops the T axis.
 * - `dt` is the storage type of q, k, v, b, w and dO (GDN2_F32 or GDN2_BF16).
 *   log_alpha, every state, o and every gradient are always fp32.
 * - Gates are post-activation values; gradients are with respect to the
 *   tensors as passed. Nothing is clamped or range-checked; q is not scaled.
 * - Supported sizes: Dk, Dv in {16, 32, 64, 128}; chunk in {16, 32, 64};
 *   B, H >= 1; T >= 0 (T = 0 writes S_final = S0 and nothing else). A ragged
 *   last chunk is handled exactly. The chunk size tiles the recurrence and
 *   does not change its result. With fp32 inputs at Dk = 128 and chunk 64
 *   the backward, the training pair and the single-pass forward run 32-token
 *   chunks inside (their LDS does not hold 64): the workspace and records
 *   sizes are those of chunk 32 (gdn2_workspace_bytes(GDN2_OP_FWD, ...) is
 *   large enough for both forwards), chunk_states keep the caller's chunk,
 *   and the backward recomputes the chunk-32 entry states instead of reading
 *   the caller's chunk_states.
 * - Numerics: fp32 inputs are computed with fp32 matrix-core products. bf16
 *   inputs use fp16 matrix-core operands for the value-side products and a
 *   two-term bf16 split for the decay-scaled key Gram matrices, always with
 *   fp32 accumulation and an fp32 state.
 *   Decay range: any log_alpha <= 0 is exact, -inf (a channel reset)
 *   included. The chunked calls floor each token's log_alpha at -20 (a decay
 *   factor of at least exp(-20) ~ 2.1e-9 per token, below fp32 resolution
 *   next to any term of order one); decode applies exp(log_alpha) as given.
 *   Chunks where some channel's cumulative log-decay from the chunk middle
 *   exceeds 60 in magnitude take a slower exact path (decay factors taken
 *   per 16-token block, the diagonal blocks pair by pair); the others a fast
 *   one. Both give the same results to rounding.
 *   Magnitudes: the bf16 backward multiplies dO and dS_final, per (batch row
 *   or sequence, head), by the power of two that brings their largest
 *   magnitude into [1, 2) (a pre-pass over dO), and every gradient back on its
 *   store, so the fp16 operand range does not limit the upstream gradients'
 *   scale; the forward's fp16 operands hold v, w*v, T (w*v) (also stored as
 *   fp16 between the two stages), U and the state, whose products must stay
 *   within fp16's range (|v| and |S0| up to 2^12 are tested).
 * - Results are deterministic (no floating-point atomics): identical inputs
 *   give bitwise identical outputs.
 * - A nullable input means zeros; a nullable output means "not written".
 * - Errors are returned as a negative gdn2_status; nothing is launched when a
 *   call returns an error detected on the host. GDN2_ERR_HIP reports a failed
 *   kernel launch (hipGetLastError after the launch).
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN2_OK = 0,
  GDN2_ERR_NULL = -1,        /* a required pointer is NULL */
  GDN2_ERR_SHAPE = -2,       /* a size is negative or out of range */
  GDN2_ERR_DTYPE = -3,       /* unknown dtype enum */
  GDN2_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  GDN2_ERR_UNSUPPORTED = -5, /* Dk, Dv or chunk not in the supported set */
  GDN2_ERR_WORKSPACE = -6,   /* workspace missing or smaller than gdn2_workspace_bytes */
  GDN2_ERR_HIP = -7          /* a HIP runtime call or kernel launch failed */
} gdn2_status;

typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

typedef enum { GDN2_OP_FWD = 0, GDN2_OP_DECODE = 1, GDN2_OP_BWD = 2, GDN2_OP_BWD_RECORDS = 3 } gdn2_op;

/* Flags of the _ex entry points (bitwise OR; any other bit gives GDN2_ERR_UNSUPPORTED).
 *
 * GDN2_FLAG_RAW_GATES -- fused gate front end. b, w and log_alpha carry the
 *   gates' pre-activations b_raw, w_raw, a_raw (same dtypes and layouts), and
 *   the kernels form b = sigmoid(b_raw), w = sigmoid(w_raw) and
 *   log_alpha = -softplus(a_raw) = -log(1 + exp(a_raw)) in fp32 as they load
 *   them, so no separate elementwise pass over HBM is needed. The pages leave
 *   the gate parametrisation open; this is the sigmoid erase/write gates and
 *   softplus log-decay of the workloads (b and w in [0, 1], alpha in (0, 1)).
 *   In gdn2_bwd_chunked_ex, db, dw and dlog_alpha are then the gradients with
 *   respect to b_raw, w_raw and a_raw: db * b (1 - b), dw * w (1 - w) and
 *   -dlog_alpha * sigmoid(a_raw). */
#define GDN2_FLAG_RAW_GATES 1u

/* GDN2_FLAG_SCALAR_B, _W, _DECAY -- gate granularity. The erase gate b, the
 *   write gate w, or the decay log_alpha holds one value per (token, head)
 *   instead of one per channel: layout [B,T,H] ([B,H] for decode, [1,T,H] for
 *   packed batches), broadcast over the channels inside the kernels, which
 *   read d times fewer bytes for it. The backward then returns that gate's
 *   gradient in the same [.., H] layout (the sum over the channels). The
 *   pages' reductions are these broadcasts: KDA has one scalar beta for both
 *   gates (SCALAR_B | SCALAR_W with b = w = beta), Gated DeltaNet also a
 *   scalar decay (| SCALAR_DECAY). Combines with GDN2_FLAG_RAW_GATES. */
#define GDN2_FLAG_SCALAR_B 2u
#define GDN2_FLAG_SCALAR_W 4u
#define GDN2_FLAG_SCALAR_DECAY 8u

/*
 * gdn2_fwd_chunked -- chunkwise WY forward over T tokens.
 *
 * Computes o (all T outputs) and optionally S_final = S_T and the chunk entry
 * states, by the chunkwise WY algorithm with the channel-wise decay absorbed
 * into asymmetric erase factors (arXiv 2605.22791 abstract; research-wiki
 * summary, "Key findings"): per chunk, the in-chunk cumulative log-decay g
 * (gate preprocessing), the strictly lower triangular erase Gram matrix A of
 * the decayed b*k against the inverse-decayed k, T = (I + A)^-1 by blocked
 * forward substitution, the WY factors W = T (decayed b*k) and
 * U = T (w*v) - W S, then o = (decayed q) S + (causal q-k term) U and
 * S <- Diag(exp(g_last)) S + (k decayed to the chunk end)^T U.
 *
 *   q, k, b      [B,T,H,Dk] dt      v, w [B,T,H,Dv] dt     log_alpha [B,T,H,Dk] fp32
 *   S0           [B,H,Dk,Dv] fp32, nullable (zero initial state)
 *   o            [B,T,H,Dv] fp32, required when T > 0
 *   S_final      [B,H,Dk,Dv] fp32, nullable
 *   chunk_states [B,H,NC,Dk,Dv] fp32, nullable (training mode when given)
 *   workspace    nullable. NULL selects the single-pass kernel: one workgroup
 *                per (batch, head, value tile) walks the chunks and recomputes
 *                each chunk's state-independent part in turn. Otherwise it must
 *                hold at least gdn2_workspace_bytes(GDN2_OP_FWD, ...) bytes,
 *                256-byte aligned, and the two-stage path runs: a
 *                chunk-parallel kernel writes every chunk's state-independent
 *                factors (W, T (w*v), decayed q and k, the causal q-k term,
 *                exp(g_last)) to the workspace, then a light sequential kernel
 *                carries the state through the chunks. Same arithmetic, same
 *                results up to rounding order. When gdn2_workspace_bytes returns
 *                0 for the sizes, the workspace is ignored.
 */
int gdn2_fwd_chunked(const void* q, const void* k, const void* v, const float* log_alpha,
                     const void* b, const void* w, const float* S0, float* o, float* S_final,
                     float* chunk_states, void* workspace, size_t workspace_bytes, int B, int T,
                     int H, int Dk, int Dv, int chunk, int dt, void* stream);

/* gdn2_fwd_chunked with flags (GDN2_FLAG_*); flags = 0 is gdn2_fwd_chunked. */
int gdn2_fwd_chunked_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                        const void* b, const void* w, const float* S0, float* o, float* S_final,
                        float* chunk_states, void* workspace, size_t workspace_bytes, int B, int T,
                        int H, int Dk, int Dv, int chunk, int dt, unsigned flags, void* stream);

/*
 * gdn2_decode_step -- one recurrence step per sequence, state updated in place
 * (constant-memory decoding, arXiv 2605.22791 abstract).
 *
 * Per (b, h): S~ = Diag(alpha) S; r = S~^T (b*k); p = S~^T q; u = w*v - r;
 * o = p + (k.q) u; S <- S~ + k u^T.  One read and one write of the fp32 state.
 *
 *   q, k, b  [B,H,Dk] dt     v, w [B,H,Dv] dt     log_alpha [B,H,Dk] fp32
 *   S        [B,H,Dk,Dv] fp32, in/out, required
 *   o        [B,H,Dv] fp32, required
 */
int gdn2_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                     const void* b, const void* w, float* S, float* o, int B, int H, int Dk,
                     int Dv, int dt, void* stream);

/* gdn2_decode_step with flags (GDN2_FLAG_*); flags = 0 is gdn2_decode_step. */
int gdn2_decode_step_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                        const void* b, const void* w, float* S, float* o, int B, int H, int Dk,
                        int Dv, int dt, unsigned flags, void* stream);

/*
 * gdn2_bwd_chunked -- gate-aware chunkwise backward (arXiv 2605.22791
 * abstract; aiexpert.news method paragraph).
 *
 * Gradients of L = <dO, o> + <dS_final, S_T> with respect to q, k, v,
 * log_alpha, b, w and S0. A reverse pass over the chunks carries the state
 * gradient from the last chunk to the first (and yields dS0); a chunk-parallel
 * pass forms every per-token gradient from the chunk's entry state and the
 * gradient of its exit state. The decay gradient is a reverse cumulative sum
 * inside each chunk plus rowsum(S_exit * dS_exit), which follows from the
 * operator's invariance under a rescaling of the key axis.
 *
 *   inputs as gdn2_fwd_chunked; dO [B,T,H,Dv] dt
 *   dS_final     [B,H,Dk,Dv] fp32, nullable (zero)
 *   chunk_states [B,H,NC,Dk,Dv] fp32 from gdn2_fwd_chunked on the same
 *                inputs, nullable (then recomputed into the workspace)
 *   dq, dk, db, dlog_alpha [B,T,H,Dk] fp32, dv, dw [B,T,H,Dv] fp32: required when T > 0
 *   dS0          [B,H,Dk,Dv] fp32, nullable (computed even when S0 is NULL)
 *   workspace    device scratch of at least gdn2_workspace_bytes(GDN2_OP_BWD, ...)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 */
int gdn2_bwd_chunked(const void* q, const void* k, const void* v, const float* log_alpha,
                     const void* b, const void* w, const float* S0, const void* dO,
                     const float* dS_final, const float* chunk_states, float* dq, float* dk,
                     float* dv, float* dlog_alpha, float* db, float* dw, float* dS0,
                     void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk,
                     int Dv, int chunk, int dt, void* stream);

/* gdn2_bwd_chunked with flags (GDN2_FLAG_*); flags = 0 is gdn2_bwd_chunked. With
 * GDN2_FLAG_RAW_GATES, chunk_states must come from gdn2_fwd_chunked_ex with the
 * same flag (or be NULL). */
int gdn2_bwd_chunked_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                        const void* b, const void* w, const float* S0, const void* dO,
                        const float* dS_final, const float* chunk_states, float* dq, float* dk,
                        float* dv, float* dlog_alpha, float* db, float* dw, float* dS0,
                        void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk,
                        int Dv, int chunk, int dt, unsigned flags, void* stream);

/*
 * Training pair -- the forward also writes everything the backward needs, so
 * the backward skips its own chunk-parallel record pass.
 *
 * The backward's per-chunk records (the causal q-k term, the decayed q and k,
 * W, T and the decayed b*k, in the orientation of the reverse pass) depend on
 * the inputs alone, and the forward's chunk-parallel kernel already forms every
 * factor they are made of. gdn2_fwd_chunked_train runs that kernel once for
 * both directions: it writes the forward's records to `workspace` (as
 * gdn2_fwd_chunked_ex does) and the backward's to `records`, then runs the
 * forward chain, which also stores every chunk's entry state in `records`.
 * gdn2_bwd_chunked_records then runs the reverse chain and the per-chunk
 * gradient kernel from `records`.
 *
 * The entry states are kept at the precision the backward consumes them in:
 * fp32 for fp32 inputs, fp16 for 16-bit inputs (every matrix-core product
 * that uses them rounds them to fp16 operands). Results equal those of
 * gdn2_fwd_chunked_ex followed by gdn2_bwd_chunked_ex on the same inputs bit
 * for bit, except dlog_alpha with 16-bit inputs: its rowsum(S_entry * dS_exit)
 * term then takes the fp16 entry state, a difference of at most
 * 2^-12 sum|S_entry * dS_exit| per key channel and chunk (up to 6.4e-3 of
 * rms(dlog_alpha) in the parity tests, whose initial states are large; the
 * error against the float64 oracle on a B=8 H=16 T=4096 batch is unchanged).
 *
 *   records       device buffer of at least gdn2_records_bytes(...) bytes,
 *                 256-byte aligned, owned by the caller, opaque; written by
 *                 gdn2_fwd_chunked_train, read by gdn2_bwd_chunked_records,
 *                 which must get the same inputs, sizes and flags (it does not
 *                 check: other contents give meaningless gradients)
 *   workspace     forward: gdn2_workspace_bytes(GDN2_OP_FWD, ...) bytes;
 *                 backward: gdn2_workspace_bytes(GDN2_OP_BWD_RECORDS, ...) bytes;
 *                 both 256-byte aligned, contents on entry ignored
 * Other arguments as gdn2_fwd_chunked_ex / gdn2_bwd_chunked_ex (S0 enters
 * only the forward: the first chunk's entry state in `records` is S0). Both
 * return GDN2_ERR_UNSUPPORTED for sizes the two-stage backward does not cover
 * (gdn2_records_bytes returns 0 for them).
 */
size_t gdn2_records_bytes(int B, int T, int H, int Dk, int Dv, int chunk, int dt);
int gdn2_fwd_chunked_train(const void* q, const void* k, const void* v, const float* log_alpha,
                           const void* b, const void* w, const float* S0, float* o, float* S_final,
                           void* records, size_t records_bytes, void* workspace,
                           size_t workspace_bytes, int B, int T, int H, int Dk, int Dv, int chunk,
                           int dt, unsigned flags, void* stream);
int gdn2_bwd_chunked_records(const void* q, const void* k, const void* v, const float* log_alpha,
                             const void* b, const void* w, const void* dO, const float* dS_final,
                             const void* records, size_t records_bytes, float* dq, float* dk,
                             float* dv, float* dlog_alpha, float* db, float* dw, float* dS0,
                             void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk,
                             int Dv, int chunk, int dt, unsigned flags, void* stream);

/*
 * Packed variable-length batches (the form trainers on concatenated documents
 * and serving batches use; [README] training-setup list). N sequences of
 * different lengths are packed along T of a [1, T, H, D] layout: sequence n
 * covers tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 (cu_seqlens: [N+1] int64 on
 * the device, 8-byte aligned, normally 0 = cu[0] <= ... <= cu[N] = T). Each sequence runs the recurrence from its own entry
 * state; chunks never cross a sequence boundary. The offsets are read on the
 * device only (no host synchronisation); they are first made non-decreasing
 * and clamped to [0, T], so no input can make a kernel read or write outside
 * the tensors; tokens outside [cu[0], cu[N]) are left unwritten.
 *
 *   q, k, b, log_alpha [1,T,H,Dk]; v, w, dO [1,T,H,Dv]; o and gradients likewise
 *   S0, S_final, dS_final, dS0  [N,H,Dk,Dv] fp32 (nullable as in the dense calls)
 *   chunk_states [H, gdn2_varlen_max_chunks(N,T,chunk), Dk, Dv] fp32: the entry
 *                state of every chunk, the sequences' chunks in order (entries past
 *                the last chunk are not written)
 *   workspace    gdn2_varlen_workspace_bytes(op, ...) bytes, 256-byte aligned (required)
 *   flags        GDN2_FLAG_* as for the _ex calls
 * Same kernels as the dense calls (two-stage forward, two-stage backward).
 */
int gdn2_varlen_max_chunks(int N, int T, int chunk);
size_t gdn2_varlen_workspace_bytes(int op, int N, int T, int H, int Dk, int Dv, int chunk, int dt);
int gdn2_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                    const void* b, const void* w, const long long* cu_seqlens, int N,
                    const float* S0, float* o, float* S_final, float* chunk_states,
                    void* workspace, size_t workspace_bytes, int T, int H, int Dk, int Dv,
                    int chunk, int dt, unsigned flags, void* stream);
int gdn2_bwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                    const void* b, const void* w, const long long* cu_seqlens, int N,
                    const float* S0, const void* dO, const float* dS_final,
                    const float* chunk_states, float* dq, float* dk, float* dv,
                    float* dlog_alpha, float* db, float* dw, float* dS0, void* workspace,
                    size_t workspace_bytes, int T, int H, int Dk, int Dv, int chunk, int dt,
                    unsigned flags, void* stream);

/*
 * Training pair for packed batches: gdn2_fwd_varlen_train / gdn2_bwd_varlen_records
 * are gdn2_fwd_chunked_train / gdn2_bwd_chunked_records (see there: one record
 * pass for both directions, entry states kept in `records`, fp16 for 16-bit
 * inputs) over the packed layout of gdn2_fwd_varlen / gdn2_bwd_varlen.
 *   records    gdn2_varlen_records_bytes(...) bytes, 256-byte aligned, opaque;
 *              both calls need the same cu_seqlens, inputs, sizes and flags
 *   workspace  forward: gdn2_varlen_workspace_bytes(GDN2_OP_FWD, ...);
 *              backward: gdn2_varlen_workspace_bytes(GDN2_OP_BWD_RECORDS, ...)
 * Results equal gdn2_fwd_varlen + gdn2_bwd_varlen bit for bit, except
 * dlog_alpha with 16-bit inputs (as for the dense pair).
 */
size_t gdn2_varlen_records_bytes(int N, int T, int H, int Dk, int Dv, int chunk, int dt);
int gdn2_fwd_varlen_train(const void* q, const void* k, const void* v, const float* log_alpha,
                          const void* b, const void* w, const long long* cu_seqlens, int N,
                          const float* S0, float* o, float* S_final, void* records,
                          size_t records_bytes, void* workspace, size_t workspace_bytes, int T,
                          int H, int Dk, int Dv, int chunk, int dt, unsigned flags, void* stream);
int gdn2_bwd_varlen_records(const void* q, const void* k, const void* v, const float* log_alpha,
                            const void* b, const void* w, const long long* cu_seqlens, int N,
                            const void* dO, const float* dS_final, const void* records,
                            size_t records_bytes, float* dq, float* dk, float* dv,
                            float* dlog_alpha, float* db, float* dw, float* dS0, void* workspace,
                            size_t workspace_bytes, int T, int H, int Dk, int Dv, int chunk, int dt,
                            unsigned flags, void* stream);

/*
 * gdn2_decode_step_slots -- one decode step for B sequences whose states live
 * in a pool: entry b uses S_pool[slots[b]] ([num_slots, H, Dk, Dv] fp32, in
 * place); slots [B] int32 on the device. An entry whose slot is negative or
 * >= num_slots has no state: its o is set to zero and nothing else is touched.
 * Entries must name distinct slots (two entries on one slot race).
 */
int gdn2_decode_step_slots(const void* q, const void* k, const void* v, const float* log_alpha,
                           const void* b, const void* w, float* S_pool, const int* slots,
                           int num_slots, float* o, int B, int H, int Dk, int Dv, int dt,
                           unsigned flags, void* stream);

/* Workspace bytes an entry point needs for these sizes: the backward's
 * requirement, the forward's two-stage path (0 when that path does not cover
 * the sizes), 0 for decode. Returns 0 for invalid sizes as well; the call
 * itself reports them. */
size_t gdn2_workspace_bytes(int op, int B, int T, int H, int Dk, int Dv, int chunk, int dt);

/*
 * gdn2_fwd_chunked_noalloc -- gdn2_fwd_chunked's two-stage path for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc): the workspace is a device array owned by the
 * library, GDN2_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the first
 * load of the library's device code until the process ends. Arguments as
 * gdn2_fwd_chunked without the workspace pair; results are identical to
 * gdn2_fwd_chunked with a workspace (the same kernels).
 *
 * Sizes whose forward workspace, gdn2_workspace_bytes(GDN2_OP_FWD, ...), exceeds
 * GDN2_NOALLOC_SCRATCH_BYTES return GDN2_ERR_WORKSPACE before any device work;
 * sizes that need no workspace run the single-pass kernel. The call allocates
 * nothing: its first call on a device only looks up that device's copy of the
 * array (with that device current). Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (concurrent streams, threads) race
 * and must be ordered by the caller; nothing in the array needs to be cleared.
 */
#define GDN2_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int gdn2_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                             const void* b, const void* w, const float* S0, float* o, float* S_final,
                             float* chunk_states, int B, int T, int H, int Dk, int Dv, int chunk,
                             int dt, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* gdn2_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int gdn2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
