// Per-call sequence table for the chunkwise forward, built on the device so
// that cu_seqlens never has to be copied to the host.
//
//   seq_start[n], seq_len[n]   token range of sequence n: [P_n, P_{n+1}) with
//                              P_i = clamp(max(cu[0..i]), 0, T), so ranges never
//                              overlap and the lengths sum to at most T whatever
//                              the offsets hold (offsets that decrease give
//                              empty sequences instead of overlapping ones)
//   chunk_off[0..N]            exclusive prefix sum of ceil(len / 64)
//   order[r]                   sequences by decreasing length (ties: lower
//                              index first) so the longest serial chains start
//                              first; identity when lengths are uniform or N is
//                              large (the quadratic ranking is then skipped)
#include "ckda_internal.h"

namespace ckda {
namespace {

constexpr int kThreads = 256;
constexpr int kRankMax = 1024;   // rank-sort sequences only up to this many

__global__ __launch_bounds__(kThreads) void seq_table_kernel(const int32_t *__restrict__ cu,
                                                             int B, int T, int N, SeqTable tab) {
  __shared__ int32_t s_part[kThreads + 1];
  const int t = threadIdx.x;
  // Each thread owns a contiguous segment [lo, hi) of the sequences.
  const int per = (N + kThreads - 1) / kThreads;
  const int lo = min(t * per, N), hi = min(lo + per, N);
  if (!cu) {
    for (int n = lo; n < hi; ++n) {
      tab.seq_start[n] = n * T;
      tab.seq_len[n] = T;
    }
  } else {
    // Offsets made monotone: P_i = clamp(max(cu[0..i]), 0, T).  The running
    // maximum is scanned per segment, then across segments through LDS.
    int32_t m = 0;                       // every P_i is >= 0
    for (int n = lo; n < hi; ++n) m = max(m, cu[n]);
    s_part[t + 1] = m;
    if (t == 0) s_part[0] = 0;
    __syncthreads();
    if (t == 0)
      for (int i = 1; i <= kThreads; ++i) s_part[i] = max(s_part[i], s_part[i - 1]);
    __syncthreads();
    int32_t run = s_part[t];             // max of cu[0 .. lo - 1] (and 0)
    for (int n = lo; n < hi; ++n) {
      run = max(run, cu[n]);
      const int32_t p0 = min(run, T);
      const int32_t p1 = min(max(run, cu[n + 1]), T);
      tab.seq_start[n] = p0;
      tab.seq_len[n] = p1 - p0;
    }
    __syncthreads();                     // s_part is reused below
  }
  __syncthreads();

  // chunk_off: each thread scans its segment, then the segment sums.
  int32_t sum = 0;
  for (int n = lo; n < hi; ++n) sum += (tab.seq_len[n] + kChunk - 1) / kChunk;
  s_part[t + 1] = sum;
  if (t == 0) s_part[0] = 0;
  __syncthreads();
  if (t == 0)
    for (int i = 1; i <= kThreads; ++i) s_part[i] += s_part[i - 1];
  __syncthreads();
  int32_t acc = s_part[t];
  for (int n = lo; n < hi; ++n) {
    tab.chunk_off[n] = acc;
    acc += (tab.seq_len[n] + kChunk - 1) / kChunk;
  }
  if (t == kThreads - 1) tab.chunk_off[N] = s_part[kThreads];

  // order: longest first.
  const bool rank = cu != nullptr && N <= kRankMax;
  for (int i = t; i < N; i += kThreads) {
    if (!rank) {
      tab.order[i] = i;
      continue;
    }
    const int li = tab.seq_len[i];
    int r = 0;
    for (int j = 0; j < N; ++j) {
      const int lj = tab.seq_len[j];
      r += (lj > li) || (lj == li && j < i);
    }
    tab.order[r] = i;
  }
}

// Debug aid: fill a buffer with the all-ones bit pattern, a quiet NaN as fp32
// and as fp64, so that any read of a value no kernel wrote shows up as NaN.
__global__ __launch_bounds__(kThreads) void poison_kernel(uint32_t *__restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kThreads)
    p[i] = 0xFFFFFFFFu;
}

}  // namespace

hipError_t launch_poison(void *buf, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(poison_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(kThreads), 0, stream, static_cast<uint32_t *>(buf), n);
  return hipGetLastError();
}

hipError_t launch_seq_table(const int32_t *cu_seqlens, int B, int T, int N, SeqTable tab,
                            hipStream_t stream) {
  hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, B, T, N,
                     tab);
  return hipGetLastError();
}

}  // namespace ckda
