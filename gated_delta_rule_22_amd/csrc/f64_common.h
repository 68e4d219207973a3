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
  static constexpr size_t TI = 0;                 // T^T, T = (I + A)^-1 [C][C]
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

// --------------------------------------------------------------------------
// Block product on the fp64 matrix cores, v_mfma_f64_16x16x4_f64:
// Out(m, n) = sum_{kk < K} A(m, kk) B(kk, n) for m < 64, n < NB, by NT (256
// or 512) threads, with no LDS staging and no barrier inside: fa and fb are
// called in the instruction's operand layout, fa (typically global memory)
// PF 16-deep K-slices ahead of the multiply, fb (typically LDS) one slice ahead.  The output is cut into 16 x 16
// tiles; wave w takes row block w % 4 and column blocks (w / 4) TPW + jj
// (jj < TPW).  The caller reads its results through MOwn: accumulator
// element acc[jj][r] is Out(MOwn::row(r), MOwn::col(jj)).  Operand layout of
// the instruction (one lane l, one K step of 4): A(l % 16, l / 16) and
// B(l / 16, l % 16); result tile element (4 r + l / 16, l % 16) in
// accumulator r.  Within a slice lane l takes K indices 4 (l / 16) + q for
// q < 4 (any fixed permutation of K is the same sum), so that each lane reads
// four consecutive K of one row of A.
typedef double d4 __attribute__((ext_vector_type(4)));

template <int NB, int NT = kThreads>
struct MOwn {
  static_assert(NT == 256 || NT == 512, "256 or 512 threads");
  static constexpr int TPW = NB / 16 / (NT / 256);     // column tiles per wave
  static_assert(TPW >= 1 && NB % 16 == 0, "NB must be a multiple of 16 * NT / 256");
  __device__ static int row(int r) {
    return 16 * ((threadIdx.x >> 6) & 3) + 4 * r + ((threadIdx.x & 63) >> 4);
  }
  __device__ static int col(int jj) {
    return 16 * ((threadIdx.x >> 8) * TPW + jj) + (threadIdx.x & 15);
  }
};

// A left operand whose rows are contiguous in K can be wrapped as a Quad:
// f(m, k0) returns A(m, k0 .. k0 + 3) from one or two wide loads, where the
// plain form makes four.
template <typename F4>
struct Quad {
  F4 f;
};
template <typename F4>
__device__ __forceinline__ Quad<F4> quad(F4 f) {
  return Quad<F4>{f};
}
template <typename T>
struct IsQuad {
  static constexpr bool value = false;
};
template <typename F4>
struct IsQuad<Quad<F4>> {
  static constexpr bool value = true;
};
// Four consecutive doubles (16-byte aligned) and four consecutive floats
// (16-byte aligned) as a d4.
__device__ __forceinline__ d4 ld4d(const double *p) {
  const double2 a = *reinterpret_cast<const double2 *>(p), b = *reinterpret_cast<const double2 *>(p + 2);
  return d4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ d4 ld4f(const float *p) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  return d4{a.x, a.y, a.z, a.w};
}

// The left operand's slices in flight: mgemm_start issues the first PF of
// them, mgemm_run multiplies.  A kernel may call mgemm_start early (before a
// barrier, or before the previous product's epilogue) when the left operand
// does not depend on what happens in between.
template <int PF = 3>
struct ARing {
  double r[PF + 1][4];
};

template <int PF = 3, typename FA>
__device__ __forceinline__ void mgemm_start(const FA &fa, ARing<PF> &ring) {
  const int l = threadIdx.x & 63;
  const int m = 16 * ((threadIdx.x >> 6) & 3) + (l & 15);
  const int kq = 4 * (l >> 4);
#pragma unroll
  for (int b = 0; b < PF; ++b) {
    if constexpr (IsQuad<FA>::value) {
      const d4 x = fa.f(m, 16 * b + kq);
#pragma unroll
      for (int q = 0; q < 4; ++q) ring.r[b][q] = x[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) ring.r[b][q] = fa(m, 16 * b + kq + q);
    }
  }
}

template <int NB, int K, int NT = kThreads, int PF = 3, bool ZERO = true, typename FA,
          typename FB>
__device__ __forceinline__ void mgemm_run(const FA &fa, const FB &fb, ARing<PF> &ring,
                                          d4 (&acc)[MOwn<NB, NT>::TPW]) {
  constexpr int TPW = MOwn<NB, NT>::TPW;
  constexpr int NS = K / 16;              // K-slices
  constexpr int RING = PF + 1;            // A-operand slices held in registers
  static_assert(K % 16 == 0 && NS % RING == 0, "K must be a multiple of 16 (PF + 1)");
  static_assert(RING % 2 == 0, "B's two-slice rotation is indexed by the slice's parity");
  const int l = threadIdx.x & 63;
  const int m = 16 * ((threadIdx.x >> 6) & 3) + (l & 15);
  const int n0 = 16 * ((threadIdx.x >> 8) * TPW) + (l & 15);
  const int kq = 4 * (l >> 4);
  auto load = [&](int s, double (&a)[4]) {
    if constexpr (IsQuad<FA>::value) {
      const d4 x = fa.f(m, 16 * s + kq);
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = x[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = fa(m, 16 * s + kq + q);
    }
  };
  if (ZERO) {                              // else accumulate onto acc
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) acc[jj] = d4{0.0, 0.0, 0.0, 0.0};
  }
  // A's slice s is loaded PF slices before it is multiplied, B's one slice
  // before (B is typically in LDS)
  double rb[2][4][TPW];
  auto loadb = [&](int s, double (&bb)[4][TPW]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) bb[q][jj] = fb(16 * s + kq + q, n0 + 16 * jj);
  };
  loadb(0, rb[0]);
#pragma unroll 1
  for (int s0 = 0; s0 < NS; s0 += RING) {
#pragma unroll
    for (int b = 0; b < RING; ++b) {
      if (s0 + b + PF < NS) load(s0 + b + PF, ring.r[(b + PF) % RING]);
      if (s0 + b + 1 < NS) loadb(s0 + b + 1, rb[(b + 1) & 1]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj)
          acc[jj] = __builtin_amdgcn_mfma_f64_16x16x4f64(ring.r[b][q], rb[b & 1][q][jj], acc[jj],
                                                         0, 0, 0);
    }
  }
}

template <int NB, int K, int NT = kThreads, int PF = 3, bool ZERO = true, typename FA,
          typename FB>
__device__ __forceinline__ void mgemm(const FA &fa, const FB &fb,
                                      d4 (&acc)[MOwn<NB, NT>::TPW]) {
  ARing<PF> ring;
  mgemm_start<PF>(fa, ring);
  mgemm_run<NB, K, NT, PF, ZERO>(fa, fb, ring, acc);
}

// Sum over 16 consecutive lanes (16 g .. 16 g + 15): the lanes that hold one
// row of an mgemm result tile.
__device__ __forceinline__ double sum16(double x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Workgroups are dealt to the eight XCDs in turn.  For a grid of
// round_up(rows, 8) * nv workgroups, xcd_block gives this workgroup's row and
// column block so that the nv column blocks of one row run on the same XCD and
// share its L2 (they read the same per-chunk records).  False past the last row.
__device__ __forceinline__ bool xcd_block(int nv, int rows, int &row, int &jb) {
  const unsigned wg = blockIdx.x, local = wg >> 3;
  jb = (int)(local % (unsigned)nv);
  row = (int)((local / (unsigned)nv) * 8 + (wg & 7));
  return row < rows;
}
__host__ __forceinline__ unsigned xcd_grid(int nv, int rows) {
  return (unsigned)(((rows + 7) / 8) * 8 * nv);
}

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
