// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stddef.h>
#include <stdint.h>

#include "ckda.h"

namespace ckda {

constexpr int kChunk = 64;          // tokens per chunk of the chunkwise forward

// ---------------------------------------------------------------- input loads
// q, k, v arrive as bf16 or fp32; both widen exactly to fp32 (and fp64).
__device__ __forceinline__ float to_f32(__hip_bfloat16 x) { return __bfloat162float(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
// Four consecutive elements (8-byte aligned for bf16, 16-byte for fp32) as fp32.
__device__ __forceinline__ float4 load4_f32(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ float4 load4_f32(const __hip_bfloat16 *p) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

// ---------------------------------------------------------------- schedule
// Per-call sequence table, computed on the device from cu_seqlens (or the
// uniform B x T layout) into the workspace:
//   seq_start[n], seq_len[n]  token offset and length of sequence n
//   chunk_off[n]              first flat chunk index of sequence n (N+1 entries)
//   order[r]                  sequence index of rank r, longest first
struct SeqTable {
    int32_t *seq_start;
    int32_t *seq_len;
    int32_t *chunk_off;
    int32_t *order;
};

// Workspace layout for a forward call (host-side arithmetic only).
struct FwdLayout {
    size_t table_bytes;      // the SeqTable arrays, 256-byte aligned
    size_t rec_bytes;        // fp64 path: bytes of one (chunk, head) record
    size_t n_chunks_ub;      // upper bound of chunks over all sequences
    size_t total;            // total workspace bytes
};
FwdLayout fwd_layout(int B, int T, int H, int dk, int dv, int N, int in_dtype);
SeqTable seq_table(void *workspace, int N);

hipError_t launch_seq_table(const int32_t *cu_seqlens, int B, int T, int N, SeqTable tab,
                            hipStream_t stream);
// Fills `bytes` (a multiple of 4; 4-byte aligned) with a NaN bit pattern.
hipError_t launch_poison(void *buf, size_t bytes, hipStream_t stream);

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *S, float *o, int N, int H, int dk, int dv,
                         int in_dtype, hipStream_t stream);

// fp64 chunkwise forward (fp32 inputs).
hipError_t launch_fwd_f64(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *S0, int T_rows, int H, int dk, int dv,
                          int N, int in_dtype, SeqTable tab, size_t n_chunks_ub, void *records,
                          size_t rec_bytes, void *o, float *S_T, int signed_gates, int l2norm,
                          int o_bf16, hipStream_t stream);

// Fused bf16 chunkwise forward on matrix cores (bf16 inputs).
// signed_gates = 0 is KDA mode: the gates' signs are ignored (|g| is used).
// l2norm: q and k are L2-normalised per (token, head) inside the kernel.
// o_bf16: o is bfloat16 (else fp32).
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                           int dk, int dv, int N, SeqTable tab, int packed, int signed_gates,
                           int l2norm, int o_bf16, hipStream_t stream);

// The same forward as two kernels (uniform rows, no fused options): a
// preparation kernel writes every prepared 16-token block's slot image to
// `img` (fwd_bf16_split_bytes bytes), then a state kernel loads them.  Kept to
// measure the hand-off the fused kernel replaced; results are bit-identical.
size_t fwd_bf16_split_bytes(int T, int H, int dk, int N);
hipError_t launch_fwd_bf16_split(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *S0, void *o, float *S_T, int T,
                                 int H, int dk, int dv, int N, SeqTable tab, int signed_gates,
                                 void *img, hipStream_t stream);

// fp64 chunkwise backward (both input dtypes).  Runs the records and the
// forward's serial pass (keeping per-chunk states and U), the reverse pass of
// the state gradient, then the per-chunk gradients.  signed_gates = 0 is KDA
// mode (|g| is used; the gradient with respect to g is then dlog|g| / g, the
// same formula).  l2norm: q and k are L2-normalised per (token, head) before
// use, and their gradients pass back through that normalisation.
size_t f64_bwd_scratch_bytes(int dk, int dv);
hipError_t launch_bwd_f64(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *S0, const float *dO, const float *dS_T,
                          int H, int dk, int dv, int N, int in_dtype, SeqTable tab,
                          size_t n_chunks_ub, void *records, size_t rec_bytes, double *S_chunks,
                          double *U_chunks, double *dU_chunks, double *dSe_chunks,
                          double *scratch, float *dq, float *dk_out, float *dv_out, float *dg,
                          float *dbeta, float *dS0, int signed_gates, int l2norm,
                          hipStream_t stream);

}  // namespace ckda
