// Pieces shared by the fp64 chunkwise kernels (forward records and backward).
#pragma once

#include "ckda_internal.h"

namespace ckda {
namespace f64 {

constexpr int kThreads = 256;
constexpr int C = kChunk;
constexpr int kBV = 32;               // dv columns per serial-pass workgroup
constexpr double kLog2Floor = -1000.0;  // log2|alpha| is floored here (alpha = 0)

// Record of one (chunk, head), written by the record kernel: offsets in doubles.
// With the per-channel gate ratio r_ij = prod_{j<s<=i} alpha_s and
// gamma_i = prod_{s<=i} alpha_s inside the chunk:
template <int DK, int DV>
struct Rec {
  static constexpr size_t TI = 0;                 // T = (I + A)^-1     [C][C]
  static constexpr size_t P = TI + C * C;         // P (lower incl.)    [C][C]
  static constexpr size_t AH = P + C * C;         // A / beta (strict)  [C][C]
  static constexpr size_t W = AH + C * C;         // W                  [C][DK]
  static constexpr size_t UB = W + C * DK;        // Ubar               [C][DV]
  static constexpr size_t QT = UB + C * DV;       // gamma * Q          [C][DK]
  static constexpr size_t KH = QT + C * DK;       // K * gamma_n/gamma  [C][DK]
  static constexpr size_t GK = KH + C * DK;       // gamma * K          [C][DK]
  static constexpr size_t GN = GK + C * DK;       // gamma_n            [DK]
  static constexpr size_t SIZE = GN + DK;
};

__device__ __forceinline__ int find_seq(const int32_t *chunk_off, int N, int c) {
  int lo = 0, hi = N;          // chunk_off[lo] <= c < chunk_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace f64

size_t f64_record_bytes(int dk, int dv);

// Records of every (chunk, head), then the serial chunk pass over the states.
// o and S_T may be NULL (not written).  S_chunks [chunk][H][dk][dv] receives
// the state entering every chunk and U_chunks [chunk][H][C][dv] the chunk's
// new values U = Ubar - W S (both fp64, NULL = not written).
hipError_t launch_f64_pass(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, int H, int dk, int dv, int N,
                           int in_dtype, SeqTable tab, size_t n_chunks_ub, void *records,
                           size_t rec_bytes, void *o, float *S_T, int signed_gates, int l2norm,
                           int o_bf16, double *S_chunks, double *U_chunks, hipStream_t stream);

}  // namespace ckda
