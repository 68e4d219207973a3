// Chunkwise CKDA forward computed in fp64 (the fp32-input path).
//
// The chunked algebra follows from unrolling the update rule (blog post "One
// update, one quarter turn", ELI5 "The mirror") inside a chunk of C = 64
// tokens with incoming state S.  With the per-channel gate ratio
// r_ij = prod_{j<s<=i} alpha_s (r_ii = 1) and gamma_i = prod_{s<=i} alpha_s:
//
//   A_ij  = beta_i sum_c k_ic r_ij,c k_jc   (i > j),   T = (I + A)^-1
//   W     = T Diag(beta) (gamma * K),       Ubar = T Diag(beta) V
//   P_ij  = sum_c q_ic r_ij,c k_jc          (j <= i)
//   U     = Ubar - W S
//   O     = (gamma * Q) S + P U
//   S'    = Diag(gamma_n) S + (K * gamma_n / gamma)^T U
//
// Signed gates (CKDA summary, "Methodology in Plain English": gate magnitudes
// live in log space, so the sign is kept apart): every ratio is formed as
// (-1)^(pi_i xor pi_j) * 2^(G_i - G_j) from the in-chunk inclusive cumulative
// sum G of log2|alpha| and the cumulative parity pi of negative gates.
//
// Two kernels, with the S-independent work stored per (chunk, head) in the
// workspace:
//   f64_intra  grid (chunks, heads): G, pi, A and P (element by element, so
//              every ratio is <= 1 in magnitude and nothing can overflow),
//              T by forward substitution, then W, Ubar, gamma*Q, K_hat, gamma_n.
//              T and A / beta stay in the record for the backward pass.
//   f64_inter  grid (dv blocks x sequences x heads): the serial chunk loop on
//              an fp64 state slice held in LDS; for the backward pass it can
//              also keep the state entering each chunk and the chunk's U.
// This path favours clarity and fp64 accuracy (fp32 inputs carry a 1e-5
// relative tolerance) over speed; bf16 inputs use the matrix-core path.
#include "f64_common.h"

namespace ckda {
namespace {

using namespace f64;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kThreads) void f64_intra(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, int H, int N, SeqTable tab,
    double *__restrict__ records, size_t rec_doubles, int signed_gates, int l2norm) {
  using R = Rec<DK, DV>;
  __shared__ double s_G[C * DK];        // log2-magnitude cumsum; later reused for T
  __shared__ float s_k[C * DK];
  __shared__ uint8_t s_par[C * DK];
  __shared__ double s_A[C * (C + 1)];
  __shared__ double s_beta[C];
  __shared__ double s_fq[C];            // query normalisation factor per token (1 if off)

  const int cflat = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (cflat >= tab.chunk_off[N]) return;
  const int n = find_seq(tab.chunk_off, N, cflat);
  const int lc = cflat - tab.chunk_off[n];
  const int t0 = tab.seq_start[n] + lc * C;
  const int nt = min(C, tab.seq_len[n] - lc * C);
  double *rec = records + ((size_t)cflat * H + h) * rec_doubles;

  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };   // token-head row

  // ---- gates: inclusive cumsum of log2|alpha| and parity of negatives.
  if (t < DK) {
    double G = 0.0;
    uint8_t par = 0;
    for (int i = 0; i < C; ++i) {
      float a = 1.f, kk = 0.f;
      if (i < nt) {
        a = g[row(i) * DK + t];
        kk = to_f32(k[row(i) * DK + t]);
      }
      G += fmax(log2(fabs((double)a)), kLog2Floor);
      par ^= (uint8_t)(signed_gates && a < 0.f);   // KDA mode: signs ignored
      s_G[i * DK + t] = G;
      s_par[i * DK + t] = par;
      s_k[i * DK + t] = kk;
    }
  }
  if (t < C) s_beta[t] = t < nt ? (double)beta[row(t)] : 0.0;
  __syncthreads();
  // ---- optional L2 normalisation of q and k per token: (sum x^2 + 1e-6)^(-1/2)
  if (t < C) {
    double fk = 1.0, fq = 1.0;
    if (l2norm && t < nt) {
      double sk = 1e-6, sq = 1e-6;
      for (int c = 0; c < DK; ++c) {
        const double kk = s_k[t * DK + c], qq = to_f32(q[row(t) * DK + c]);
        sk += kk * kk;
        sq += qq * qq;
      }
      fk = 1.0 / sqrt(sk);
      fq = 1.0 / sqrt(sq);
    }
    s_fq[t] = fq;
    if (l2norm)
      for (int c = 0; c < DK; ++c) s_k[t * DK + c] = (float)(s_k[t * DK + c] * fk);
  }
  __syncthreads();

  // ---- A (strictly lower) and P (lower incl. diagonal), element by element.
  for (int p = t; p < C * C; p += kThreads) {
    const int i = p / C, j = p % C;
    double accA = 0.0, accP = 0.0;
    if (j <= i && i < nt) {
      const TIn *qi = q + row(i) * DK;
      for (int c = 0; c < DK; ++c) {
        const double r = ((s_par[i * DK + c] ^ s_par[j * DK + c]) ? -1.0 : 1.0) *
                         exp2(s_G[i * DK + c] - s_G[j * DK + c]);
        const double rk = r * (double)s_k[j * DK + c];
        accA += (double)s_k[i * DK + c] * rk;
        accP += (double)to_f32(qi[c]) * rk;
      }
      accP *= s_fq[i];
    }
    s_A[i * (C + 1) + j] = (j < i) ? s_beta[i] * accA : 0.0;
    rec[R::AH + p] = (j < i) ? accA : 0.0;
    rec[R::P + p] = accP;
  }

  // ---- gamma-scaled operands (masked tokens have k = q = 0).
  for (int p = t; p < C * DK; p += kThreads) {
    const int i = p / DK, c = p % DK;
    const double Gi = s_G[i * DK + c], Gn = s_G[(C - 1) * DK + c];
    const double si = s_par[i * DK + c] ? -1.0 : 1.0;
    const double sn = (s_par[i * DK + c] ^ s_par[(C - 1) * DK + c]) ? -1.0 : 1.0;
    const double gam = si * exp2(Gi);
    const double kk = s_k[p];
    const double qq = i < nt ? (double)to_f32(q[row(i) * DK + c]) * s_fq[i] : 0.0;
    rec[R::QT + p] = qq * gam;
    rec[R::GK + p] = kk * gam;
    rec[R::KH + p] = kk * sn * exp2(Gn - Gi);
    if (i == C - 1) rec[R::GN + c] = gam;
  }
  __threadfence();
  __syncthreads();

  // ---- T = (I + A)^-1 by forward substitution; column j per thread.
  double *s_T = s_G;     // G is dead; T is C x (C+1)
  if (t < C) {
    const int j = t;
    for (int i = 0; i < C; ++i) s_T[i * (C + 1) + j] = (i == j) ? 1.0 : 0.0;
    for (int i = j + 1; i < C; ++i) {
      double s = 0.0;
      for (int m = j; m < i; ++m) s += s_A[i * (C + 1) + m] * s_T[m * (C + 1) + j];
      s_T[i * (C + 1) + j] = -s;
    }
  }
  __syncthreads();

  // ---- T, W = T Diag(beta) (gamma*K), Ubar = T Diag(beta) V.
  for (int p = t; p < C * C; p += kThreads) {
    const int i = p / C, j = p % C;
    rec[R::TI + p] = s_T[i * (C + 1) + j];
  }
  for (int p = t; p < C * DK; p += kThreads) {
    const int i = p / DK, c = p % DK;
    double acc = 0.0;
    for (int j = 0; j <= i; ++j) acc += s_T[i * (C + 1) + j] * s_beta[j] * rec[R::GK + j * DK + c];
    rec[R::W + p] = acc;
  }
  for (int p = t; p < C * DV; p += kThreads) {
    const int i = p / DV, c = p % DV;
    double acc = 0.0;
    for (int j = 0; j <= i && j < nt; ++j)
      acc += s_T[i * (C + 1) + j] * s_beta[j] * (double)to_f32(v[row(j) * DV + c]);
    rec[R::UB + p] = acc;
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void f64_inter(
    const float *__restrict__ S0, int H, int N, SeqTable tab, const double *__restrict__ records,
    size_t rec_doubles, void *__restrict__ o, float *__restrict__ S_T, int o_bf16,
    double *__restrict__ S_chunks, double *__restrict__ U_chunks) {
  using R = Rec<DK, DV>;
  __shared__ double s_S[DK * kBV];
  __shared__ double s_U[C * kBV];

  constexpr int NV = DV / kBV;
  const int jb = blockIdx.x % NV, rh = blockIdx.x / NV, t = threadIdx.x;
  const int n = tab.order[rh / H], h = rh % H;
  const int len = tab.seq_len[n], start = tab.seq_start[n];
  const int nch = (len + C - 1) / C;
  const size_t sbase = ((size_t)n * H + h) * DK * DV + (size_t)jb * kBV;

  for (int p = t; p < DK * kBV; p += kThreads) {
    const int c = p / kBV, j = p % kBV;
    s_S[p] = S0 ? (double)S0[sbase + (size_t)c * DV + j] : 0.0;
  }
  __syncthreads();

  for (int lc = 0; lc < nch; ++lc) {
    const size_t ch = (size_t)(tab.chunk_off[n] + lc) * H + h;
    const double *rec = records + ch * rec_doubles;
    const int nt = min(C, len - lc * C);
    if (S_chunks)
      for (int p = t; p < DK * kBV; p += kThreads)
        S_chunks[ch * DK * DV + (size_t)(p / kBV) * DV + jb * kBV + p % kBV] = s_S[p];
    // U = Ubar - W S
    for (int p = t; p < C * kBV; p += kThreads) {
      const int i = p / kBV, j = p % kBV;
      double acc = rec[R::UB + i * DV + jb * kBV + j];
      for (int c = 0; c < DK; ++c) acc -= rec[R::W + i * DK + c] * s_S[c * kBV + j];
      s_U[p] = acc;
      if (U_chunks) U_chunks[ch * C * DV + (size_t)i * DV + jb * kBV + j] = acc;
    }
    __syncthreads();
    // O = (gamma Q) S + P U
    for (int p = t; p < C * kBV && o; p += kThreads) {
      const int i = p / kBV, j = p % kBV;
      if (i >= nt) continue;
      double acc = 0.0;
      for (int c = 0; c < DK; ++c) acc += rec[R::QT + i * DK + c] * s_S[c * kBV + j];
      for (int m = 0; m <= i; ++m) acc += rec[R::P + i * C + m] * s_U[m * kBV + j];
      const size_t oi = ((size_t)(start + lc * C + i) * H + h) * DV + jb * kBV + j;
      if (o_bf16)
        static_cast<__hip_bfloat16 *>(o)[oi] = __float2bfloat16((float)acc);
      else
        static_cast<float *>(o)[oi] = (float)acc;
    }
    __syncthreads();
    // S' = Diag(gamma_n) S + K_hat^T U
    for (int p = t; p < DK * kBV; p += kThreads) {
      const int c = p / kBV, j = p % kBV;
      double acc = rec[R::GN + c] * s_S[p];
      for (int m = 0; m < nt; ++m) acc += rec[R::KH + m * DK + c] * s_U[m * kBV + j];
      s_S[p] = acc;
    }
    __syncthreads();
  }
  if (S_T)
    for (int p = t; p < DK * kBV; p += kThreads) {
      const int c = p / kBV, j = p % kBV;
      S_T[sbase + (size_t)c * DV + j] = (float)s_S[p];
    }
}

template <typename TIn, int DK, int DV>
hipError_t launch_shape(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *S0, int H, int N, SeqTable tab,
                        size_t n_chunks_ub, void *records, size_t rec_bytes, void *o,
                        float *S_T, int signed_gates, int l2norm, int o_bf16,
                        double *S_chunks, double *U_chunks, hipStream_t stream) {
  const size_t rec_doubles = rec_bytes / sizeof(double);
  if (n_chunks_ub > 0) {
    hipLaunchKernelGGL((f64_intra<TIn, DK, DV>), dim3((unsigned)n_chunks_ub, H), dim3(kThreads),
                       0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                       static_cast<const TIn *>(v), g, beta, H, N, tab,
                       static_cast<double *>(records), rec_doubles, signed_gates, l2norm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((f64_inter<DK, DV>), dim3((DV / kBV) * N * H), dim3(kThreads), 0, stream, S0,
                     H, N, tab, static_cast<const double *>(records), rec_doubles, o, S_T, o_bf16,
                     S_chunks, U_chunks);
  return hipGetLastError();
}

}  // namespace

size_t f64_record_bytes(int dk, int dv) {
  return sizeof(double) * (3 * (size_t)C * C + 4 * (size_t)C * dk + (size_t)C * dv + dk);
}

hipError_t launch_f64_pass(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, int H, int dk, int dv, int N,
                           int in_dtype, SeqTable tab, size_t n_chunks_ub, void *records,
                           size_t rec_bytes, void *o, float *S_T, int signed_gates, int l2norm,
                           int o_bf16, double *S_chunks, double *U_chunks, hipStream_t stream) {
#define CKDA_F64_CASE(TIN, DK_, DV_)                                                           \
  if (dk == DK_ && dv == DV_)                                                                  \
    return launch_shape<TIN, DK_, DV_>(q, k, v, g, beta, S0, H, N, tab, n_chunks_ub, records, \
                                       rec_bytes, o, S_T, signed_gates, l2norm, o_bf16,       \
                                       S_chunks, U_chunks, stream);
  if (in_dtype == CKDA_BF16) {
    CKDA_F64_CASE(__hip_bfloat16, 64, 64)
    CKDA_F64_CASE(__hip_bfloat16, 64, 128)
    CKDA_F64_CASE(__hip_bfloat16, 128, 64)
    CKDA_F64_CASE(__hip_bfloat16, 128, 128)
  } else {
    CKDA_F64_CASE(float, 64, 64)
    CKDA_F64_CASE(float, 64, 128)
    CKDA_F64_CASE(float, 128, 64)
    CKDA_F64_CASE(float, 128, 128)
  }
#undef CKDA_F64_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f64(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *S0, int T_rows, int H, int dk, int dv,
                          int N, int in_dtype, SeqTable tab, size_t n_chunks_ub, void *records,
                          size_t rec_bytes, void *o, float *S_T, int signed_gates, int l2norm,
                          int o_bf16, hipStream_t stream) {
  (void)T_rows;
  return launch_f64_pass(q, k, v, g, beta, S0, H, dk, dv, N, in_dtype, tab, n_chunks_ub, records,
                         rec_bytes, o, S_T, signed_gates, l2norm, o_bf16, nullptr, nullptr,
                         stream);
}

}  // namespace ckda
