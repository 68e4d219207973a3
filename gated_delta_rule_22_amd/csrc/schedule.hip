// Per-call sequence table for the chunkwise forward, built on the device so
// that cu_seqlens never has to be copied to the host.
//
//   seq_start[n], seq_len[n]   token range of sequence n (clamped into [0, T])
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
  for (int n = t; n < N; n += kThreads) {
    int s, e;
    if (cu) {
      s = min(max(cu[n], 0), T);
      e = min(max(cu[n + 1], s), T);
    } else {
      s = n * T;
      e = s + T;
    }
    tab.seq_start[n] = s;
    tab.seq_len[n] = e - s;
  }
  __syncthreads();

  // chunk_off: each thread scans a contiguous segment, then the segment sums.
  const int per = (N + kThreads - 1) / kThreads;
  const int lo = min(t * per, N), hi = min(lo + per, N);
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

}  // namespace

hipError_t launch_seq_table(const int32_t *cu_seqlens, int B, int T, int N, SeqTable tab,
                            hipStream_t stream) {
  hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, B, T, N,
                     tab);
  return hipGetLastError();
}

}  // namespace ckda
