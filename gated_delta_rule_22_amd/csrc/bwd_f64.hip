// Chunkwise CKDA backward, computed in fp64.
//
// Gradient of L = sum(dO * o) + sum(dS_T * S_T) for the recurrence of the
// blog post "One update, one quarter turn" (ELI5, "The mirror") with the
// readout o_t = S_t^T q_t, through the chunk algebra of the forward (names as
// in the record of f64_common.h; inside a chunk with incoming state S):
//
//   U  = T X,  X = Diag(beta) (V - (gamma*K) S),  T = (I + A)^-1
//   O  = (gamma*Q) S + P U
//   S' = Diag(gamma_n) S + KH^T U
//
// Reverse mode, given dO and dS' (the gradient reaching the chunk's end):
//
//   dU = KH dS' + P^T dO
//   dS = Diag(gamma_n) dS' + (gamma*Q)^T dO - W^T dU         (to the previous chunk)
//   dX = T^T dU,  dV = Diag(beta) dX,  dP = tril(dO U^T),  dA = -strict_tril(dX U^T)
//   dbeta_i = dX_i . V_i - (gamma*K)_i . (dX S^T)_i + sum_j (A/beta)_ij dA_ij
//
// and the key, query and gate gradients collect, per (token i, channel c), the
// direct terms from gamma*Q, gamma*K and KH and the pair terms from A and P,
// each of which carries the ratio r_ij = gamma_i / gamma_j.  Because every
// term depends on the gates only through the in-chunk log-magnitudes
// Gamma_i = sum_{s<=i} ln|alpha_s|, the gradient with respect to Gamma_i is
// the sum of those terms weighted +1 where Gamma_i appears in a numerator and
// -1 in a denominator; then dln|alpha_s| = sum_{i>=s} dGamma_i (a reverse
// cumulative sum inside the chunk) and dalpha_s = dln|alpha_s| / alpha_s.  The
// gate signs are piecewise constant and carry no gradient.
//
// Kernels (all arithmetic fp64; gradients are written as fp32):
//   records and the forward's serial pass  (fwd_f64.hip), keeping the state
//              entering every chunk and every chunk's U;
//   f64_bwd_state  grid (dv blocks x sequences x heads): the reverse serial
//              pass over chunks for dS, writing dU and dS' of every chunk and
//              dS0;
//   f64_bwd_chunk  grid (chunks, heads): everything else, one chunk per
//              workgroup, with the dense products as LDS-staged block products
//              (f64_common.h) and the ratio-weighted pair sums channel group by
//              channel group.
#include "f64_common.h"

namespace ckda {
namespace {

using namespace f64;

// --------------------------------------------------------------------------
// f64_bwd_state: reverse serial pass of dS over the chunks of one
// (sequence, head, kBV-column block), the products on the fp64 matrix cores
// with their right operands (dS', dO, dU) in LDS.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void f64_bwd_state(
    const float *__restrict__ dO, const float *__restrict__ dS_T, int H, int N, SeqTable tab,
    const double *__restrict__ records, size_t rec_doubles, double *__restrict__ dU_chunks,
    double *__restrict__ dSe_chunks, float *__restrict__ dS0) {
  using R = Rec<DK, DV>;
  using Own = MOwn<kBV>;
  constexpr int TPW = Own::TPW;
  __shared__ double s_dS[DK * kBV];
  __shared__ double s_dO[C * kBV];
  __shared__ double s_dU[C * kBV];

  constexpr int NV = DV / kBV;
  const int jb = blockIdx.x % NV, rh = blockIdx.x / NV, t = threadIdx.x;
  const int n = tab.order[rh / H], h = rh % H;
  const int len = tab.seq_len[n], start = tab.seq_start[n];
  const int nch = (len + C - 1) / C;
  const size_t sbase = ((size_t)n * H + h) * DK * DV + (size_t)jb * kBV;

  for (int p = t; p < DK * kBV; p += kThreads) {
    const int c = p / kBV, j = p % kBV;
    s_dS[p] = dS_T ? (double)dS_T[sbase + (size_t)c * DV + j] : 0.0;
  }
  for (int lc = nch - 1; lc >= 0; --lc) {
    const size_t ch = (size_t)(tab.chunk_off[n] + lc) * H + h;
    const double *rec = records + ch * rec_doubles;
    const int nt = min(C, len - lc * C);
    for (int p = t; p < C * kBV; p += kThreads) {
      const int i = p / kBV, j = p % kBV;
      s_dO[p] = i < nt ? (double)dO[((size_t)(start + lc * C + i) * H + h) * DV + jb * kBV + j]
                       : 0.0;
    }
    __syncthreads();         // dS' and dO complete
    for (int p = t; p < DK * kBV; p += kThreads)
      dSe_chunks[ch * DK * DV + (size_t)(p / kBV) * DV + jb * kBV + p % kBV] = s_dS[p];
    // dU = KH dS' + P^T dO, as one product over [dS'; dO]
    {
      d4 acc[TPW];
      mgemm<kBV, DK + C>(
          [&](int m, int kk) {
            return kk < DK ? rec[R::KH + m * DK + kk] : rec[R::P + (kk - DK) * C + m];
          },
          [&](int kk, int nn) {
            return kk < DK ? s_dS[kk * kBV + nn] : s_dO[(kk - DK) * kBV + nn];
          },
          acc);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = Own::row(r), j = Own::col(jj);
          s_dU[i * kBV + j] = acc[jj][r];
          dU_chunks[ch * C * DV + (size_t)i * DV + jb * kBV + j] = acc[jj][r];
        }
    }
    __syncthreads();         // dU complete; every read of dS' done
    // dS = Diag(gamma_n) dS' + (gamma Q)^T dO - W^T dU, 64 state rows at a time
    // (in place: the product reads dO and dU only)
#pragma unroll
    for (int half = 0; half < DK / 64; ++half) {
      d4 acc[TPW];
      mgemm<kBV, 2 * C>(
          [&](int m, int kk) {
            return kk < C ? rec[R::QT + kk * DK + half * 64 + m]
                          : -rec[R::W + (kk - C) * DK + half * 64 + m];
          },
          [&](int kk, int nn) { return kk < C ? s_dO[kk * kBV + nn] : s_dU[(kk - C) * kBV + nn]; },
          acc);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = half * 64 + Own::row(r), j = Own::col(jj);
          s_dS[c * kBV + j] = rec[R::GN + c] * s_dS[c * kBV + j] + acc[jj][r];
        }
    }
    __syncthreads();         // dS complete; dO and dU free
  }
  if (dS0)
    for (int p = t; p < DK * kBV; p += kThreads) {
      const int c = p / kBV, j = p % kBV;
      dS0[sbase + (size_t)c * DV + j] = (float)s_dS[p];
    }
}

// Per-chunk scratch (doubles): dX [C][DV]; G, sign and the direct parts of
// dq, dk and dGamma, each [C][DK].
template <int DK, int DV>
struct Scr {
  static constexpr size_t DX = 0;
  static constexpr size_t G = DX + C * DV;
  static constexpr size_t SG = G + C * DK;
  static constexpr size_t AQ = SG + C * DK;
  static constexpr size_t AK = AQ + C * DK;
  static constexpr size_t AG = AK + C * DK;
  static constexpr size_t SIZE = AG + C * DK;
};

constexpr int kCG = 16;                  // channels per group in the pair sums
constexpr int kTri = C * (C + 1) / 2;    // packed lower triangle (incl. diagonal)
__device__ __forceinline__ int tri(int i, int j) { return i * (i + 1) / 2 + j; }   // j <= i

// --------------------------------------------------------------------------
// f64_bwd_chunk: all per-chunk gradients of one (chunk, head).
// The chunk-gradient kernel runs 512 threads (two waves per SIMD) over the
// same LDS, so that each wave holds half the rows of every block product.
constexpr int kBT = 512;
constexpr int kRPT = 1024 / kBT;          // rows per thread in the block products

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kBT) void f64_bwd_chunk(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ dO,
    int H, int N, SeqTable tab, const double *__restrict__ records, size_t rec_doubles,
    const double *__restrict__ S_chunks, const double *__restrict__ U_chunks,
    const double *__restrict__ dU_chunks, const double *__restrict__ dSe_chunks,
    double *__restrict__ scratch, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta, int signed_gates,
    int l2norm) {
  using R = Rec<DK, DV>;
  using X = Scr<DK, DV>;
  constexpr int NBM = DV > 64 ? DV : 64;
  constexpr int kStage = stage_doubles(NBM);
  constexpr int kGroup = 8 * C * kCG > C * DK * 3 / 2 ? 8 * C * kCG : C * DK * 3 / 2;
  __shared__ double s_P[kTri];            // dP (lower incl.), packed
  __shared__ double s_DA[kTri];           // beta_i dA_ij (strictly lower; diagonal 0), packed
  __shared__ double s_u[kStage > kGroup ? kStage : kGroup];  // staging | group operands
  __shared__ double s_ag[C * kCG];
  __shared__ double s_beta[C], s_db[C];
  __shared__ double s_R[DK];
  __shared__ int s_fb[DK];
  __shared__ double s_red[(kBT / 64) * DK], s_red2[2 * DK], s_dGn[DK];
  __shared__ double s_fk[C], s_fq[C];     // key/query normalisation factors per token (1 if off)
  __shared__ double s_kd[C], s_qd[C];     // khat . dkhat and qhat . dqhat per token

  const int cflat = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (cflat >= tab.chunk_off[N]) return;
  const int n = find_seq(tab.chunk_off, N, cflat);
  const int lc = cflat - tab.chunk_off[n];
  const int t0 = tab.seq_start[n] + lc * C;
  const int nt = min(C, tab.seq_len[n] - lc * C);
  const size_t ch = (size_t)cflat * H + h;
  const double *rec = records + ch * rec_doubles;
  const double *Sc = S_chunks + ch * DK * DV;
  const double *dSe = dSe_chunks + ch * DK * DV;
  const double *Uc = U_chunks + ch * C * DV;
  const double *dUc = dU_chunks + ch * C * DV;
  double *scr = scratch + ch * X::SIZE;
  const int rgp = t >> 4, cl = t & 15, wave = t >> 6;
  double *sA = s_u, *sB = s_u + kStageA;

  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };   // token-head row
  auto dO_at = [&](int m, int c) { return m < nt ? (double)dO[row(m) * DV + c] : 0.0; };
  auto gam_at = [&](int m, int c) {
    return scr[X::SG + m * DK + c] * exp2(scr[X::G + m * DK + c]);
  };

  // ---- phase 0: in-chunk gate log-magnitudes and signs: log2|alpha| for
  // every (token, channel) in parallel into LDS (the sign rides in the sign
  // bit of a float copy of alpha), then the scans per channel.
  double *s_l = s_u;                                   // [C][DK] log2|alpha|
  float *s_sg = reinterpret_cast<float *>(s_u + C * DK); // [C][DK] alpha (sign only)
#pragma unroll 4
  for (int p = t; p < C * DK; p += kBT) {
    const float a = p / DK < nt ? g[row(p / DK) * DK + p % DK] : 1.f;
    s_l[p] = fmax(log2(fabs((double)a)), kLog2Floor);
    s_sg[p] = a;
  }
  __syncthreads();
  if (t < DK) {
    double G = 0.0, gmax = 0.0, gmin = 0.0;
    bool par = false;
#pragma unroll 8
    for (int i = 0; i < C; ++i) {
      const float a = s_sg[i * DK + t];
      G += s_l[i * DK + t];
      par ^= (signed_gates && a < 0.f);   // KDA mode: signs ignored
      gmax = fmax(gmax, G);
      gmin = fmin(gmin, G);
      scr[X::G + i * DK + t] = G;
      scr[X::SG + i * DK + t] = par ? -1.0 : 1.0;
    }
    // The pair sums form r_ij = e_i f_j with e = sign 2^(G - Rm), f = sign 2^(Rm - G)
    // about the midpoint Rm of the channel's range; beyond +-1000 binary orders
    // that product could leave fp64's range, and the channel takes exp2 per pair.
    s_R[t] = 0.5 * (gmax + gmin);
    s_fb[t] = (gmax - gmin) > 2000.0;
  }
  if (t < C) {
    s_beta[t] = t < nt ? (double)beta[row(t)] : 0.0;
    s_db[t] = 0.0;
    s_kd[t] = 0.0;
    s_qd[t] = 0.0;
  }
  // optional q/k normalisation factors (sum x^2 + 1e-6)^(-1/2): four threads per
  // token, 32 channels each
  {
    const int i = t >> 2, part = t & 3;
    double sk = 0.0, sq = 0.0;
    if (l2norm && i < nt) {
#pragma unroll 8
      for (int c = part * (DK / 4); c < (part + 1) * (DK / 4); ++c) {
        const double kk = to_f32(k[row(i) * DK + c]), qq = to_f32(q[row(i) * DK + c]);
        sk += kk * kk;
        sq += qq * qq;
      }
    }
    sk += __shfl_xor(sk, 1);
    sk += __shfl_xor(sk, 2);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if (part == 0 && i < C) {
      s_fk[i] = (l2norm && i < nt) ? 1.0 / sqrt(sk + 1e-6) : 1.0;
      s_fq[i] = (l2norm && i < nt) ? 1.0 / sqrt(sq + 1e-6) : 1.0;
    }
  }
  __threadfence_block();   // scratch is read back by this workgroup only
  __syncthreads();

  // ---- phase 1: dX = T^T dU; dV = Diag(beta) dX; dbeta += dX_i . V_i
  {
    double acc[kRPT][DV / 16];
    gemm64<DV, C, true, false, kBT>(
        sA, sB, [&](int m, int kk) { return rec[R::TI + kk * C + m]; },
        [&](int kk, int nn) { return dUc[kk * DV + nn]; }, acc);
#pragma unroll
    for (int r = 0; r < kRPT; ++r) {
      const int m = rgp * kRPT + r;
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < DV / 16; ++jj) {
        const int nn = cl + 16 * jj;
        scr[X::DX + m * DV + nn] = acc[r][jj];
        if (m < nt) {
          dv[row(m) * DV + nn] = (float)(s_beta[m] * acc[r][jj]);
          part += acc[r][jj] * (double)to_f32(v[row(m) * DV + nn]);
        }
      }
      part = sum16(part);
      if (cl == 0) s_db[m] += part;
    }
  }
  __threadfence_block();   // scratch is read back by this workgroup only
  __syncthreads();

  // ---- phase 2: dP = tril(dO U^T) and beta_i dA_ij, dA = -strict_tril(dX U^T)
  {
    double acc[kRPT][4];
    gemm64<64, DV, false, true, kBT>(
        sA, sB, dO_at, [&](int kk, int nn) { return Uc[nn * DV + kk]; }, acc);
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = rgp * kRPT + r, j = cl + 16 * jj;
        if (j <= m) s_P[tri(m, j)] = acc[r][jj];
      }
    gemm64<64, DV, false, true, kBT>(
        sA, sB, [&](int m, int kk) { return scr[X::DX + m * DV + kk]; },
        [&](int kk, int nn) { return Uc[nn * DV + kk]; }, acc);
#pragma unroll
    for (int r = 0; r < kRPT; ++r) {
      const int m = rgp * kRPT + r;
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = cl + 16 * jj;
        const double dA = j < m ? -acc[r][jj] : 0.0;
        if (j <= m) s_DA[tri(m, j)] = s_beta[m] * dA;
        part += rec[R::AH + m * C + j] * dA;
      }
      part = sum16(part);
      if (cl == 0) s_db[m] += part;
    }
  }

  // ---- phase 3: the direct parts, 64 channels at a time, kept in registers
  // over the three products and stored once.
#pragma unroll 1
  for (int hf = 0; hf < DK / 64; ++hf) {
    const int cb = hf * 64;
    double aq[kRPT][4], ak[kRPT][4], ag[kRPT][4], gam[kRPT][4], acc[kRPT][4];
    // dQT = dO S^T: dq = gamma dQT; dGamma = q gamma dQT
    gemm64<64, DV, false, true, kBT>(
        sA, sB, dO_at, [&](int kk, int nn) { return Sc[(cb + nn) * DV + kk]; }, acc);
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = rgp * kRPT + r, c = cb + cl + 16 * jj;
        gam[r][jj] = gam_at(m, c);
        aq[r][jj] = gam[r][jj] * acc[r][jj];
        ag[r][jj] = rec[R::QT + m * DK + c] * acc[r][jj];
      }
    // M5 = dX S^T: d(gamma K) = -Diag(beta) M5
    gemm64<64, DV, false, true, kBT>(
        sA, sB, [&](int m, int kk) { return scr[X::DX + m * DV + kk]; },
        [&](int kk, int nn) { return Sc[(cb + nn) * DV + kk]; }, acc);
#pragma unroll
    for (int r = 0; r < kRPT; ++r) {
      const int m = rgp * kRPT + r;
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = cb + cl + 16 * jj;
        const double gk = rec[R::GK + m * DK + c];
        ak[r][jj] = -s_beta[m] * gam[r][jj] * acc[r][jj];
        ag[r][jj] -= s_beta[m] * gk * acc[r][jj];
        part -= gk * acc[r][jj];
      }
      part = sum16(part);
      if (cl == 0) s_db[m] += part;
    }
    // dKH = U dS'^T: dk += (gamma_n / gamma) dKH; dGamma_i -= k (gamma_n/gamma) dKH,
    // and the same amount, summed over i, goes to dGamma_n.
    gemm64<64, DV, false, true, kBT>(
        sA, sB, [&](int m, int kk) { return Uc[m * DV + kk]; },
        [&](int kk, int nn) { return dSe[(cb + nn) * DV + kk]; }, acc);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = cb + cl + 16 * jj;
      const double Gn = scr[X::G + (C - 1) * DK + c], sn = scr[X::SG + (C - 1) * DK + c];
      double col = 0.0;
#pragma unroll
      for (int r = 0; r < kRPT; ++r) {
        const int m = rgp * kRPT + r;
        const double khr = scr[X::SG + m * DK + c] * sn * exp2(Gn - scr[X::G + m * DK + c]);
        const double term = rec[R::KH + m * DK + c] * acc[r][jj];
        ak[r][jj] += khr * acc[r][jj];
        ag[r][jj] -= term;
        col += term;
      }
      col += __shfl_xor(col, 16);
      col += __shfl_xor(col, 32);
      if ((t & 63) < 16) s_red[wave * DK + c] = col;
    }
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = rgp * kRPT + r, c = cb + cl + 16 * jj;
        scr[X::AQ + m * DK + c] = aq[r][jj];
        scr[X::AK + m * DK + c] = ak[r][jj];
        scr[X::AG + m * DK + c] = ag[r][jj];
      }
  }
  // gamma_n sum_j dS'[c][j] S[c][j]: two threads per channel
  for (int p = t; p < 2 * DK; p += kBT) {
    const int c = p % DK, half = p / DK;
    double part = 0.0;
#pragma unroll 16
    for (int j = half * (DV / 2); j < (half + 1) * (DV / 2); ++j)
      part += dSe[c * DV + j] * Sc[c * DV + j];
    s_red2[half * DK + c] = part;
  }
  __threadfence_block();   // scratch is read back by this workgroup only
  __syncthreads();
  for (int c = t; c < DK; c += kBT)
  {
    double col = 0.0;
#pragma unroll
    for (int w = 0; w < kBT / 64; ++w) col += s_red[w * DK + c];
    s_dGn[c] = col + rec[R::GN + c] * (s_red2[c] + s_red2[DK + c]);
  }

  // ---- phase 4: pair sums per group of kCG channels, then the gate gradients
  const int gcl = t % kCG, grw = t / kCG;          // channel in the group, row slot
  constexpr int kRowSlots = kBT / kCG;
  // this thread's gates, keys and queries of the next channel group, loaded
  // while the current group is summed
  constexpr int NG = C * kCG / kBT;
  float pg[NG], pk[NG], pq[NG];
  auto load_group = [&](int c0) {
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int p = t + u * kBT, i = p / kCG, cc = c0 + p % kCG;
      pg[u] = i < nt ? g[row(i) * DK + cc] : 1.f;
      pk[u] = i < nt ? to_f32(k[row(i) * DK + cc]) : 0.f;
      pq[u] = i < nt ? to_f32(q[row(i) * DK + cc]) : 0.f;
    }
  };
  load_group(0);
  for (int c0 = 0; c0 < DK; c0 += kCG) {
    const int c = c0 + gcl;
    double *e = s_u, *f = s_u + C * kCG, *kk_ = s_u + 2 * C * kCG, *qq = s_u + 3 * C * kCG;
    double *ra = s_u + 4 * C * kCG;       // 1 / alpha (floored magnitude)
    double *saq = s_u + 5 * C * kCG, *sak = s_u + 6 * C * kCG, *sag = s_u + 7 * C * kCG;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int p = t + u * kBT, i = p / kCG, cc = c0 + p % kCG;
      const double G = scr[X::G + i * DK + cc], sg = scr[X::SG + i * DK + cc];
      {
        const double floor_mag = exp2(kLog2Floor);
        const double a = pg[u];
        ra[p] = 1.0 / (fabs(a) < floor_mag ? (a < 0.0 ? -floor_mag : floor_mag) : a);
      }
      if (s_fb[cc]) {
        e[p] = G;
        f[p] = sg;
      } else {
        e[p] = sg * exp2(G - s_R[cc]);
        f[p] = sg * exp2(s_R[cc] - G);
      }
      kk_[p] = pk[u] * s_fk[i];
      qq[p] = pq[u] * s_fq[i];
      saq[p] = scr[X::AQ + i * DK + cc];
      sak[p] = scr[X::AK + i * DK + cc];
      sag[p] = scr[X::AG + i * DK + cc];
    }
    __syncthreads();
    if (c0 + kCG < DK) load_group(c0 + kCG);
    {
      const bool fb = s_fb[c];
#pragma unroll 1
      for (int u = 0; u < C / kRowSlots; ++u) {
        const int i = grw + kRowSlots * u;
        double R1 = 0.0, R2 = 0.0, C1 = 0.0, C2 = 0.0;
        const double ei = e[i * kCG + gcl], fi = f[i * kCG + gcl];
        const double *Pi = s_P + tri(i, 0), *DAi = s_DA + tri(i, 0);
        // row i: sum over j <= i of dP_ij k_j r_ij and (beta dA)_ij k_j r_ij;
        // column i: sum over m >= i of (beta dA)_mi k_m r_mi and dP_mi q_m r_mi.
        if (!fb) {
          // four independent partial sums per quantity keep the FMA chains short
          double r1[4] = {0.0, 0.0, 0.0, 0.0}, r2[4] = {0.0, 0.0, 0.0, 0.0};
          int j = 0;
          for (; j + 3 <= i; j += 4) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const double kr = kk_[(j + w) * kCG + gcl] * (ei * f[(j + w) * kCG + gcl]);
              r1[w] = fma(Pi[j + w], kr, r1[w]);
              r2[w] = fma(DAi[j + w], kr, r2[w]);
            }
          }
          for (; j <= i; ++j) {
            const double kr = kk_[j * kCG + gcl] * (ei * f[j * kCG + gcl]);
            r1[0] = fma(Pi[j], kr, r1[0]);
            r2[0] = fma(DAi[j], kr, r2[0]);
          }
          R1 = (r1[0] + r1[1]) + (r1[2] + r1[3]);
          R2 = (r2[0] + r2[1]) + (r2[2] + r2[3]);
          double c1[4] = {0.0, 0.0, 0.0, 0.0}, c2[4] = {0.0, 0.0, 0.0, 0.0};
          int m = i;
          for (; m + 3 < C; m += 4) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const double r = e[(m + w) * kCG + gcl] * fi;
              c1[w] = fma(s_DA[tri(m + w, i)], kk_[(m + w) * kCG + gcl] * r, c1[w]);
              c2[w] = fma(s_P[tri(m + w, i)], qq[(m + w) * kCG + gcl] * r, c2[w]);
            }
          }
          for (; m < C; ++m) {
            const double r = e[m * kCG + gcl] * fi;
            c1[0] = fma(s_DA[tri(m, i)], kk_[m * kCG + gcl] * r, c1[0]);
            c2[0] = fma(s_P[tri(m, i)], qq[m * kCG + gcl] * r, c2[0]);
          }
          C1 = (c1[0] + c1[1]) + (c1[2] + c1[3]);
          C2 = (c2[0] + c2[1]) + (c2[2] + c2[3]);
        } else {                          // e holds G and f the sign
          for (int j = 0; j <= i; ++j) {
            const double r = fi * f[j * kCG + gcl] * exp2(ei - e[j * kCG + gcl]);
            const double kr = kk_[j * kCG + gcl] * r;
            R1 = fma(Pi[j], kr, R1);
            R2 = fma(DAi[j], kr, R2);
          }
          for (int m = i; m < C; ++m) {
            const double r = f[m * kCG + gcl] * fi * exp2(e[m * kCG + gcl] - ei);
            C1 = fma(s_DA[tri(m, i)], kk_[m * kCG + gcl] * r, C1);
            C2 = fma(s_P[tri(m, i)], qq[m * kCG + gcl] * r, C2);
          }
        }
        const double ki = kk_[i * kCG + gcl], qi = qq[i * kCG + gcl];
        const double gq = saq[i * kCG + gcl] + R1;
        const double gk = sak[i * kCG + gcl] + R2 + C1 + C2;
        double gG = sag[i * kCG + gcl] + qi * R1 + ki * (R2 - C1 - C2);
        if (i == C - 1) gG += s_dGn[c];
        s_ag[i * kCG + gcl] = gG;
        if (l2norm) {
          // gradients with respect to the normalised rows; the normalisation's
          // Jacobian is applied once every channel is done
          scr[X::AQ + i * DK + c] = gq;
          scr[X::AK + i * DK + c] = gk;
          const double dqd = sum16(qi * gq), dkd = sum16(ki * gk);
          if (gcl == 0) {
            s_qd[i] += dqd;
            s_kd[i] += dkd;
          }
        } else if (i < nt) {
          dq[row(i) * DK + c] = (float)gq;
          dk[row(i) * DK + c] = (float)gk;
        }
      }
    }
    __syncthreads();
    // dln|alpha_s| = sum_{i >= s} dGamma_i; dalpha = dln|alpha| / alpha
    if (t < kCG) {
      const int cc = c0 + t;
      double acc2 = 0.0;
#pragma unroll 8
      for (int i = C - 1; i >= 0; --i) {
        acc2 += s_ag[i * kCG + t];
        if (i < nt) dg[row(i) * DK + cc] = (float)(acc2 * ra[i * kCG + t]);
      }
    }
  }
  __threadfence_block();   // scratch is read back by this workgroup only
  __syncthreads();
  if (l2norm) {
    // x = xhat / f_x with xhat = x f_x:  dx = f_x (dxhat - xhat (xhat . dxhat))
#pragma unroll 4
    for (int p = t; p < nt * DK; p += kBT) {
      const int i = p / DK, c = p % DK;
      const double qh = to_f32(q[row(i) * DK + c]) * s_fq[i];
      const double kh = to_f32(k[row(i) * DK + c]) * s_fk[i];
      dq[row(i) * DK + c] = (float)(s_fq[i] * (scr[X::AQ + p] - qh * s_qd[i]));
      dk[row(i) * DK + c] = (float)(s_fk[i] * (scr[X::AK + p] - kh * s_kd[i]));
    }
  }
  if (t < nt) dbeta[row(t)] = (float)s_db[t];
}

template <typename TIn, int DK, int DV>
hipError_t launch_bwd_shape(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *dO, const float *dS_T, int H, int N,
                            SeqTable tab, size_t n_chunks_ub, const double *records,
                            size_t rec_bytes, const double *S_chunks, const double *U_chunks,
                            double *dU_chunks, double *dSe_chunks, double *scratch, float *dq,
                            float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                            int signed_gates, int l2norm, hipStream_t stream) {
  const size_t rec_doubles = rec_bytes / sizeof(double);
  hipLaunchKernelGGL((f64_bwd_state<DK, DV>), dim3((DV / kBV) * N * H), dim3(kThreads), 0, stream,
                     dO, dS_T, H, N, tab, records, rec_doubles, dU_chunks, dSe_chunks, dS0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_chunks_ub == 0) return e;
  hipLaunchKernelGGL((f64_bwd_chunk<TIn, DK, DV>), dim3((unsigned)n_chunks_ub, H), dim3(kBT),
                     0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                     static_cast<const TIn *>(v), g, beta, dO, H, N, tab, records, rec_doubles,
                     S_chunks, U_chunks, dU_chunks, dSe_chunks, scratch, dq, dk, dv, dg, dbeta,
                     signed_gates, l2norm);
  return hipGetLastError();
}

}  // namespace

size_t f64_bwd_scratch_bytes(int dk, int dv) {
  return sizeof(double) * ((size_t)C * dv + 5 * (size_t)C * dk);
}

hipError_t launch_bwd_f64(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *S0, const float *dO, const float *dS_T,
                          int H, int dk, int dv, int N, int in_dtype, SeqTable tab,
                          size_t n_chunks_ub, void *records, size_t rec_bytes, double *S_chunks,
                          double *U_chunks, double *dU_chunks, double *dSe_chunks,
                          double *scratch, float *dq, float *dk_out, float *dv_out, float *dg,
                          float *dbeta, float *dS0, int signed_gates, int l2norm, hipStream_t stream) {
  hipError_t e = launch_f64_pass(q, k, v, g, beta, S0, H, dk, dv, N, in_dtype, tab, n_chunks_ub,
                                 records, rec_bytes, nullptr, nullptr, signed_gates, l2norm, 0, S_chunks,
                                 U_chunks, stream);
  if (e != hipSuccess) return e;
  const double *rec = static_cast<const double *>(records);
#define CKDA_BWD_CASE(TIN, DK_, DV_)                                                           \
  if (dk == DK_ && dv == DV_)                                                                  \
    return launch_bwd_shape<TIN, DK_, DV_>(q, k, v, g, beta, dO, dS_T, H, N, tab, n_chunks_ub,  \
                                           rec, rec_bytes, S_chunks, U_chunks, dU_chunks,      \
                                           dSe_chunks, scratch, dq, dk_out, dv_out, dg, dbeta, \
                                           dS0, signed_gates, l2norm, stream);
  if (in_dtype == CKDA_BF16) {
    CKDA_BWD_CASE(__hip_bfloat16, 64, 64)
    CKDA_BWD_CASE(__hip_bfloat16, 64, 128)
    CKDA_BWD_CASE(__hip_bfloat16, 128, 64)
    CKDA_BWD_CASE(__hip_bfloat16, 128, 128)
  } else {
    CKDA_BWD_CASE(float, 64, 64)
    CKDA_BWD_CASE(float, 64, 128)
    CKDA_BWD_CASE(float, 128, 64)
    CKDA_BWD_CASE(float, 128, 128)
  }
#undef CKDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ckda
