// gdn2_varlen.hip -- tables of a packed variable-length batch, built on the
// device from the caller's offsets (no host synchronisation).
//
// N sequences are packed along T: sequence n covers tokens [cu[n], cu[n+1]).
// Every sequence starts a new chunk, so chunks never mix sequences; the
// chunk-parallel kernels run over (head, global chunk) and the chain kernels
// over (sequence, head). One workgroup:
//   1. cu'[n] = min(T, max(0, cu[0..n])) -- offsets made non-decreasing within
//      [0, T], so every kernel reads inside the tensors whatever it is given;
//   2. chunk_first[n] = sum over m < n of ceil((cu'[m+1] - cu'[m]) / C);
//   3. chunk_seq[g] = the sequence of global chunk g, -1 for g >= chunk_first[N]
//      up to max_chunks = T / C + N (which bounds chunk_first[N]);
//   4. for the two-level chain (segment length L > 0): seg_first[n] = sum over
//      m < n of ceil(chunks_m / L) and seg_seq[s] = the sequence of global
//      segment s, -1 past the last up to max_segs = max_chunks / L + N.

#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int kPlanThreads = 1024;

// exclusive scan of one value per thread over the workgroup (op = max or +)
template <bool MAX>
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* sh, int64_t& total) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off *= 2) {
    const int64_t y = tid >= off ? sh[tid - off] : (MAX ? INT64_MIN : 0);
    __syncthreads();
    sh[tid] = MAX ? (y > sh[tid] ? y : sh[tid]) : sh[tid] + y;
    __syncthreads();
  }
  total = sh[kPlanThreads - 1];
  const int64_t excl = tid > 0 ? sh[tid - 1] : (MAX ? INT64_MIN : 0);
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(kPlanThreads) void gdn2_varlen_plan_kernel(const int64_t* cu_in, int N, int T, int C,
                                                                          int max_chunks, int64_t* cu_out,
                                                                          int* chunk_first, int* chunk_seq, int L,
                                                                          int max_segs, int* seg_first, int* seg_seq) {
  __shared__ int64_t sh[kPlanThreads];
  const int tid = threadIdx.x;
  // each thread owns offsets [o0, o1) of the N + 1 offsets
  const int per = (N + 1 + kPlanThreads - 1) / kPlanThreads;
  const int o0 = min(N + 1, tid * per), o1 = min(N + 1, o0 + per);
  // 1. running maximum, clamped to [0, T]
  int64_t m = INT64_MIN;
  for (int i = o0; i < o1; ++i) m = cu_in[i] > m ? cu_in[i] : m;
  int64_t tot;
  int64_t run = block_exclusive_scan<true>(m, sh, tot);
  for (int i = o0; i < o1; ++i) {
    run = cu_in[i] > run ? cu_in[i] : run;
    cu_out[i] = run < 0 ? 0 : (run > T ? T : run);
  }
  __syncthreads();
  // 2. chunks per sequence and their prefix sums (sequence n = offsets n, n + 1)
  const int s1 = min(N, o1);
  int64_t cnt = 0;
  for (int n = o0; n < s1; ++n) cnt += (cu_out[n + 1] - cu_out[n] + C - 1) / C;
  int64_t first = block_exclusive_scan<false>(cnt, sh, tot);
  for (int n = o0; n < s1; ++n) {
    chunk_first[n] = (int)first;
    first += (cu_out[n + 1] - cu_out[n] + C - 1) / C;
  }
  if (tid == 0) chunk_first[N] = (int)tot;
  __syncthreads();
  // 3. the sequence of every global chunk
  for (int n = o0; n < s1; ++n)
    for (int g = chunk_first[n]; g < chunk_first[n + 1]; ++g) chunk_seq[g] = n;
  for (int g = (int)tot + tid; g < max_chunks; g += kPlanThreads) chunk_seq[g] = -1;
  if (L <= 0) return;
  // 4. segments of L chunks inside each sequence
  int64_t scnt = 0;
  for (int n = o0; n < s1; ++n) scnt += (chunk_first[n + 1] - chunk_first[n] + L - 1) / L;
  int64_t sfirst = block_exclusive_scan<false>(scnt, sh, tot);
  for (int n = o0; n < s1; ++n) {
    seg_first[n] = (int)sfirst;
    sfirst += (chunk_first[n + 1] - chunk_first[n] + L - 1) / L;
  }
  if (tid == 0) seg_first[N] = (int)tot;
  __syncthreads();
  for (int n = o0; n < s1; ++n)
    for (int g = seg_first[n]; g < seg_first[n + 1]; ++g) seg_seq[g] = n;
  for (int g = (int)tot + tid; g < max_segs; g += kPlanThreads) seg_seq[g] = -1;
}

}  // namespace

int varlen_max_chunks(int N, int T, int C) { return T / C + N; }

// Two-level chain inside packed sequences: used, as for dense batches, only when
// there are at most 32 (sequence, head) chains of 128 value columns (the plain
// chain's four-wave workgroups cannot fill a quarter of the GPU) and the batch
// holds at least 32 chunks; L chunks per segment, sized so that the run pass
// has about 128 workgroups at T / C chunks, at least 8. Past 32 chains the
// plain chain wins although it walks the longest sequence whole: the map pass
// and the composition cost more than the walk saves unless one sequence is
// several times the others (7-document B8 H16 T4096-token training step:
// 3.22 -> 2.87 ms without segments; one 16K and four 4K documents: 3.25 ->
// 3.70 ms). The segment machinery (compose kernel) needs Dv >= 32.
int varlen_seg_len(int N, int T, int H, int Dk, int Dv, int C) {
  (void)Dk;
  const long nc = T / C;
  if (Dv < 32 || nc < 32 || (long)N * H * ((Dv + 127) / 128) > 32) return 0;
  long L = (nc * H * ((Dv + 127) / 128) + 127) / 128;
  return (int)(L < 8 ? 8 : L);
}

int varlen_max_segs(int N, int T, int C, int L) { return L > 0 ? varlen_max_chunks(N, T, C) / L + N : 0; }

size_t varlen_seg_bytes(int N, int T, int H, int Dk, int Dv, int C) {
  const int L = varlen_seg_len(N, T, H, Dk, Dv, C);
  if (L == 0) return 0;
  return (size_t)H * varlen_max_segs(N, T, C, L) * ((size_t)Dk * Dk + 2 * (size_t)Dk * Dv) * sizeof(float);
}

// Table bytes inside a workspace: cu' [N+1] int64, chunk_first [N+1] int32,
// chunk_seq [max_chunks] int32, and with segments seg_first [N+1] and seg_seq
// [max_segs] int32, each 256-byte aligned.
size_t varlen_table_bytes(int N, int T, int C, int L) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t b = al((size_t)(N + 1) * 8) + al((size_t)(N + 1) * 4) + al((size_t)varlen_max_chunks(N, T, C) * 4);
  if (L > 0) b += al((size_t)(N + 1) * 4) + al((size_t)varlen_max_segs(N, T, C, L) * 4);
  return b;
}

hipError_t launch_varlen_plan(const int64_t* cu, int N, int T, int C, int L, char* tables, Varlen& vl,
                              hipStream_t s) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = tables;
  int64_t* cu_out = reinterpret_cast<int64_t*>(p);
  p += al((size_t)(N + 1) * 8);
  int* first = reinterpret_cast<int*>(p);
  p += al((size_t)(N + 1) * 4);
  int* seq = reinterpret_cast<int*>(p);
  p += al((size_t)varlen_max_chunks(N, T, C) * 4);
  vl.cu = cu_out;
  vl.chunk_first = first;
  vl.chunk_seq = seq;
  vl.nseq = N;
  vl.max_chunks = varlen_max_chunks(N, T, C);
  vl.seg_len = L;
  vl.max_segs = varlen_max_segs(N, T, C, L);
  if (L > 0) {
    vl.seg_first = reinterpret_cast<int*>(p);
    p += al((size_t)(N + 1) * 4);
    vl.seg_seq = reinterpret_cast<int*>(p);
  }
  hipLaunchKernelGGL(gdn2_varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, cu, N, T, C, vl.max_chunks, cu_out,
                     first, seq, L, vl.max_segs, const_cast<int*>(vl.seg_first), const_cast<int*>(vl.seg_seq));
  return hipGetLastError();
}

}  // namespace gdn2
