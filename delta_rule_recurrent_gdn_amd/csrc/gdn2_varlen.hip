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
//      up to max_chunks = T / C + N (which bounds chunk_first[N]).

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
                                                                          int* chunk_first, int* chunk_seq) {
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
}

}  // namespace

int varlen_max_chunks(int N, int T, int C) { return T / C + N; }

// Table bytes inside a workspace: cu' [N+1] int64, chunk_first [N+1] int32,
// chunk_seq [max_chunks] int32, each 256-byte aligned.
size_t varlen_table_bytes(int N, int T, int C) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)(N + 1) * 8) + al((size_t)(N + 1) * 4) + al((size_t)varlen_max_chunks(N, T, C) * 4);
}

hipError_t launch_varlen_plan(const int64_t* cu, int N, int T, int C, char* tables, Varlen& vl, hipStream_t s) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  int64_t* cu_out = reinterpret_cast<int64_t*>(tables);
  int* first = reinterpret_cast<int*>(tables + al((size_t)(N + 1) * 8));
  int* seq = reinterpret_cast<int*>(tables + al((size_t)(N + 1) * 8) + al((size_t)(N + 1) * 4));
  vl.cu = cu_out;
  vl.chunk_first = first;
  vl.chunk_seq = seq;
  vl.nseq = N;
  vl.max_chunks = varlen_max_chunks(N, T, C);
  hipLaunchKernelGGL(gdn2_varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, cu, N, T, C, vl.max_chunks, cu_out,
                     first, seq);
  return hipGetLastError();
}

}  // namespace gdn2
