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
//   f64_bwd_prep, f64_bwd_pairs, f64_bwd_final  everything else, per chunk
//              (the pair kernel per 32-channel block of a chunk), with every
//              contraction on the fp64 matrix cores (f64_common.h) and the
//              ratio-weighted pair sums as dense products (see below).
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
  const int t = threadIdx.x;
  int rh, jb;
  if (!xcd_block(NV, N * H, rh, jb)) return;
  const int n = tab.order[rh / H], h = rh % H;
  const int len = tab.seq_len[n], start = tab.seq_start[n];
  const int nch = (len + C - 1) / C;
  const size_t sbase = ((size_t)n * H + h) * DK * DV + (size_t)jb * kBV;

  for (int p = t; p < DK * kBV; p += kThreads) {
    const int c = p / kBV, j = p % kBV;
    s_dS[p] = dS_T ? (double)dS_T[sbase + (size_t)c * DV + j] : 0.0;
  }
  // dO of a chunk is loaded into registers one chunk ahead of its use
  constexpr int NO = C * kBV / kThreads;
  float pre[NO];
  auto load_do = [&](int lc) {
    const int nt = min(C, len - lc * C);
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int p = t + u * kThreads, i = p / kBV, j = p % kBV;
      pre[u] = i < nt ? dO[((size_t)(start + lc * C + i) * H + h) * DV + jb * kBV + j] : 0.f;
    }
  };
  if (nch > 0) load_do(nch - 1);
  for (int lc = nch - 1; lc >= 0; --lc) {
    const size_t ch = (size_t)(tab.chunk_off[n] + lc) * H + h;
    const double *rec = records + ch * rec_doubles;
    // the left operands are records, independent of the state gradient: the
    // first slices of each product are issued ahead of the barrier before it
    auto fa_u = [&](int m, int kk) {
      return kk < DK ? rec[R::KH + m * DK + kk] : rec[R::P + (kk - DK) * C + m];
    };
    auto fa_s = [&](int half) {
      return [&, half](int m, int kk) {
        return kk < C ? rec[R::QT + kk * DK + half * 64 + m]
                      : -rec[R::W + (kk - C) * DK + half * 64 + m];
      };
    };
    // (deeper rings where K allows: a ring of PF + 1 slices must divide K / 16)
    constexpr int PFU = ((DK + C) / 16) % 6 == 0 ? 5 : 3;
    ARing<PFU> ring_u;
    ARing<7> ring_s[DK / 64];
    mgemm_start(fa_u, ring_u);
#pragma unroll
    for (int u = 0; u < NO; ++u) s_dO[t + u * kThreads] = (double)pre[u];
    if (lc > 0) load_do(lc - 1);
    __syncthreads();         // dS' and dO complete
    for (int p = t; p < DK * kBV; p += kThreads)
      dSe_chunks[ch * DK * DV + (size_t)(p / kBV) * DV + jb * kBV + p % kBV] = s_dS[p];
    // dU = KH dS' + P^T dO, as one product over [dS'; dO]
    {
      d4 acc[TPW];
      mgemm_run<kBV, DK + C, kThreads, PFU>(
          fa_u,
          [&](int kk, int nn) {
            return kk < DK ? s_dS[kk * kBV + nn] : s_dO[(kk - DK) * kBV + nn];
          },
          ring_u, acc);
      mgemm_start(fa_s(0), ring_s[0]);
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
      double gn[4];                        // gamma_n of this thread's state rows
#pragma unroll
      for (int r = 0; r < 4; ++r) gn[r] = rec[R::GN + half * 64 + Own::row(r)];
      mgemm_run<kBV, 2 * C, kThreads, 7>(
          fa_s(half),
          [&](int kk, int nn) { return kk < C ? s_dO[kk * kBV + nn] : s_dU[(kk - C) * kBV + nn]; },
          ring_s[half], acc);
      if (half + 1 < DK / 64) mgemm_start(fa_s(half + 1), ring_s[half + 1]);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = half * 64 + Own::row(r), j = Own::col(jj);
          s_dS[c * kBV + j] = gn[r] * s_dS[c * kBV + j] + acc[jj][r];
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

// The per-chunk gradients run in three kernels (all 512 or 256 threads):
//   f64_bwd_prep   (chunk, head): the gate factors, dX = T^T dU (dV, the dX.V
//                  part of dbeta), dP and beta dA (the A/beta . dA part);
//   f64_bwd_pairs  (32-channel block, chunk, head): the direct terms and the
//                  pair terms of dq, dk and dGamma for its channels, and dalpha;
//   f64_bwd_final  (chunk, head): dbeta, and the Jacobian of the fused q/k
//                  normalisation.
// Every contraction runs on the fp64 matrix cores (mgemm).  The pair terms
// use the ratio split r_ij = e_i f_j about each channel's midpoint, which turns
// them into four dense products:
//   R1 = E o (dP (F o K)),      R2 = E o ((beta dA) (F o K)),
//   C1 = F o ((beta dA)^T (E o K)),  C2 = F o (dP^T (E o Q))
// (o: elementwise; K, Q the normalised keys and queries).  A channel whose
// log-gate range is too wide for the split takes the ratios one pair at a time.
constexpr int kBT = 512;                 // threads of the prep and pair kernels
constexpr int kCH = 32;                  // channels per pair-kernel workgroup

// Per-chunk scratch (doubles), written by f64_bwd_prep and f64_bwd_pairs:
//   DX [C][DV]        dX = T^T dU
//   E [C][DK]         the ratio split e = sign(gamma) 2^(G - Rm) (G = log2|gamma|,
//                     Rm the channel's integer midpoint); on exact-path
//                     channels G itself.  The other factors follow from e:
//                     gamma = e 2^Rm, f = 1 / e, gamma_n / gamma = SIG f.
//   AQ, AK [C][DK]    the pair terms R1, R2 of exact-path channels, later the
//                     gradients with respect to the normalised q and k
//   X3, X4 [C][DK]    the pair terms C1, C2 of exact-path channels
//   DP, DA [C][C]     dP and beta dA, zero above the diagonal
//   FB, RM, SIG [DK]  1 on exact-path channels; Rm; sign(gamma_n) 2^(G_n - Rm)
//   FQ, FK [C]        the q/k normalisation factors (1 if off)
//   DB [1 + NB][C]    dbeta: the prep kernel's part, then one row per block
//   QD, KD [NB][C]    qhat . dqhat and khat . dkhat per channel block
//   SGN [C][DK]       sign of gamma, one byte each (read on exact-path channels)
template <int DK, int DV>
struct Scr {
  static constexpr int NB = DK / kCH;
  static constexpr size_t DX = 0;
  static constexpr size_t E = DX + C * DV;
  static constexpr size_t AQ = E + C * DK;
  static constexpr size_t AK = AQ + C * DK;
  static constexpr size_t X3 = AK + C * DK;
  static constexpr size_t X4 = X3 + C * DK;
  static constexpr size_t DP = X4 + C * DK;
  static constexpr size_t DA = DP + C * C;
  static constexpr size_t FB = DA + C * C;
  static constexpr size_t RM = FB + DK;
  static constexpr size_t SIG = RM + DK;
  static constexpr size_t FQ = SIG + DK;
  static constexpr size_t FK = FQ + C;
  static constexpr size_t DB = FK + C;
  static constexpr size_t QD = DB + (1 + NB) * C;
  static constexpr size_t KD = QD + NB * C;
  static constexpr size_t SGN = KD + NB * C;      // C * DK bytes
  static constexpr size_t SIZE = SGN + C * DK / 8;
};

// Row sums over a wave's 16 lanes, kept per half of the column tiles (wave
// t / 256) so that every (half, row) slot has a single writer.
__device__ __forceinline__ void add_row(double (&dst)[2][C], int i, double part) {
  part = sum16(part);
  if ((threadIdx.x & 15) == 0) dst[threadIdx.x >> 8][i] += part;
}

// --------------------------------------------------------------------------
template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kBT) void f64_bwd_prep(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ dO,
    int H, int N, SeqTable tab, const double *__restrict__ records, size_t rec_doubles,
    const double *__restrict__ U_chunks, const double *__restrict__ dU_chunks,
    double *__restrict__ scratch, float *__restrict__ dv, int signed_gates, int l2norm) {
  using R = Rec<DK, DV>;
  using X = Scr<DK, DV>;
  using OwnV = MOwn<DV, kBT>;              // C x DV results
  using OwnC = MOwn<C, kBT>;               // C x C results
  constexpr int TV = OwnV::TPW, TC = OwnC::TPW;
  constexpr int SV = DV + 1;               // padded LDS row
  constexpr int kPool = C * DK > C * SV ? C * DK : C * SV;
  // one LDS pool: the phase-0 log-gates, later the staged right operands
  __shared__ double s_b[kPool];
  __shared__ int8_t s_sg[C * DK];         // the gates' signs, then the sign of gamma
  __shared__ double s_beta[C], s_dbp[2][C];
  __shared__ double s_R[DK];
  __shared__ int s_fb[DK];

  const int cflat = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (cflat >= tab.chunk_off[N]) return;
  const int n = find_seq(tab.chunk_off, N, cflat);
  const int lc = cflat - tab.chunk_off[n];
  const int t0 = tab.seq_start[n] + lc * C;
  const int nt = min(C, tab.seq_len[n] - lc * C);
  const size_t ch = (size_t)cflat * H + h;
  const double *rec = records + ch * rec_doubles;
  const double *Uc = U_chunks + ch * C * DV;
  const double *dUc = dU_chunks + ch * C * DV;
  double *scr = scratch + ch * X::SIZE;

  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };   // token-head row
  auto dO_at = [&](int m, int c) { return m < nt ? (double)dO[row(m) * DV + c] : 0.0; };

  // ---- phase 0: in-chunk gate log-magnitudes and signs: log2|alpha| for
  // every (token, channel) in parallel into LDS (the sign rides in a float
  // copy of alpha), then the scans per channel.
  double *s_l = s_b;                                    // [C][DK] log2|alpha|
  constexpr int NGL = C * DK / kBT;
  float gpre[NGL];                                      // all gate loads issued first
#pragma unroll
  for (int u = 0; u < NGL; ++u) {
    const int p = t + u * kBT;
    gpre[u] = p / DK < nt ? g[row(p / DK) * DK + p % DK] : 1.f;
  }
#pragma unroll
  for (int u = 0; u < NGL; ++u) {
    const int p = t + u * kBT;
    const float a = gpre[u];
    s_l[p] = fmax(log2(fabs((double)a)), kLog2Floor);
    s_sg[p] = (signed_gates && a < 0.f) ? -1 : 1;   // KDA mode: signs ignored
  }
  __syncthreads();
  if (t < DK) {
    // in place: s_l becomes the running G, s_sg the sign of gamma
    double G = 0.0, gmax = 0.0, gmin = 0.0;
    bool par = false;
#pragma unroll 8
    for (int i = 0; i < C; ++i) {
      par ^= s_sg[i * DK + t] < 0;
      G += s_l[i * DK + t];
      gmax = fmax(gmax, G);
      gmin = fmin(gmin, G);
      s_l[i * DK + t] = G;
      s_sg[i * DK + t] = par ? -1 : 1;
    }
    // r_ij = e_i f_j with e = sign 2^(G - Rm), f = sign 2^(Rm - G) about the
    // midpoint Rm of the channel's range; beyond +-1000 binary orders that
    // product could leave fp64's range, and the channel takes exp2 per pair.
    // (an integer midpoint: gamma = e 2^Rm is then an exact scaling of e)
    const double Rm = rint(0.5 * (gmax + gmin));
    const int fb = (gmax - gmin) > 2000.0;
    s_R[t] = Rm;
    s_fb[t] = fb;
    scr[X::FB + t] = fb;
    scr[X::RM + t] = Rm;
    scr[X::SIG + t] = (par ? -1.0 : 1.0) * exp2(G - Rm);   // sign(gamma_n) 2^(G_n - Rm)
  }
  if (t < C) {
    s_beta[t] = t < nt ? (double)beta[row(t)] : 0.0;
    s_dbp[0][t] = s_dbp[1][t] = 0.0;
  }
  // optional q/k normalisation factors (sum x^2 + 1e-6)^(-1/2): eight threads
  // per token
  {
    const int i = t >> 3, part = t & 7;
    double sk = 0.0, sq = 0.0;
    if (l2norm && i < nt) {
#pragma unroll 4
      for (int c = part * (DK / 8); c < (part + 1) * (DK / 8); ++c) {
        const double kk = to_f32(k[row(i) * DK + c]), qq = to_f32(q[row(i) * DK + c]);
        sk += kk * kk;
        sq += qq * qq;
      }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      sk += __shfl_xor(sk, o);
      sq += __shfl_xor(sq, o);
    }
    if (part == 0 && i < C) {
      scr[X::FK + i] = (l2norm && i < nt) ? 1.0 / sqrt(sk + 1e-6) : 1.0;
      scr[X::FQ + i] = (l2norm && i < nt) ? 1.0 / sqrt(sq + 1e-6) : 1.0;
    }
  }
  __syncthreads();
  // the split factor of every (token, channel), once (G itself on exact-path
  // channels), and the sign of gamma
  int8_t *sgn8 = reinterpret_cast<int8_t *>(scr + X::SGN);
#pragma unroll 2
  for (int p = t; p < C * DK; p += kBT) {
    const int c = p % DK;
    const double G = s_l[p];
    scr[X::E + p] = s_fb[c] ? G : s_sg[p] * exp2(G - s_R[c]);
    sgn8[p] = s_sg[p];
  }
  __syncthreads();

  // ---- phase 1: dX = T^T dU; dV = Diag(beta) dX; dbeta += dX_i . V_i
  for (int p = t; p < C * DV; p += kBT) s_b[(p / DV) * SV + p % DV] = dUc[p];
  __syncthreads();
  {
    d4 acc[TV];
    mgemm<DV, C, kBT>(quad([&](int m, int kk) { return ld4d(rec + R::TI + m * C + kk); }),   // T^T
                      [&](int kk, int nn) { return s_b[kk * SV + nn]; }, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = OwnV::row(r);
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < TV; ++jj) {
        const int j = OwnV::col(jj);
        const double x = acc[jj][r];
        scr[X::DX + i * DV + j] = x;
        if (i < nt) {
          dv[row(i) * DV + j] = (float)(s_beta[i] * x);
          part += x * (double)to_f32(v[row(i) * DV + j]);
        }
      }
      add_row(s_dbp, i, part);
    }
  }
  __threadfence_block();   // scratch is read back by this workgroup
  __syncthreads();

  // ---- phase 2: dP = tril(dO U^T) and beta_i dA_ij, dA = -strict_tril(dX U^T),
  // stored as full C x C matrices (zero above the diagonal)
  for (int p = t; p < C * DV; p += kBT) s_b[(p / DV) * SV + p % DV] = Uc[p];
  __syncthreads();
  {
    auto ut = [&](int kk, int nn) { return s_b[nn * SV + kk]; };   // U^T
    d4 acc[TC];
    mgemm<C, DV, kBT>(dO_at, ut, acc);
#pragma unroll
    for (int jj = 0; jj < TC; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = OwnC::row(r), j = OwnC::col(jj);
        scr[X::DP + i * C + j] = j <= i ? acc[jj][r] : 0.0;
      }
    double ah[TC][4];                  // the epilogue's A / beta, loaded ahead
#pragma unroll
    for (int jj = 0; jj < TC; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) ah[jj][r] = rec[R::AH + OwnC::row(r) * C + OwnC::col(jj)];
    mgemm<C, DV, kBT>([&](int m, int kk) { return scr[X::DX + m * DV + kk]; }, ut, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = OwnC::row(r);
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < TC; ++jj) {
        const int j = OwnC::col(jj);
        const double dA = j < i ? -acc[jj][r] : 0.0;
        scr[X::DA + i * C + j] = s_beta[i] * dA;
        part += ah[jj][r] * dA;
      }
      add_row(s_dbp, i, part);
    }
  }
  __syncthreads();
  if (t < C) scr[X::DB + t] = s_dbp[0][t] + s_dbp[1][t];
}

// --------------------------------------------------------------------------
// One workgroup per (kCH-channel block, chunk, head).  The workgroups of one
// (chunk, head) are placed on the same XCD (workgroups are dealt to the eight
// XCDs in turn), so that the operands they share are read once into its L2.
template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kBT, 2) void f64_bwd_pairs(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const float *__restrict__ dO, int H, int N, SeqTable tab,
    const double *__restrict__ records, size_t rec_doubles, const double *__restrict__ S_chunks,
    const double *__restrict__ U_chunks, const double *__restrict__ dSe_chunks,
    double *__restrict__ scratch, size_t n_ch, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dg, int l2norm) {
  using R = Rec<DK, DV>;
  using X = Scr<DK, DV>;
  using Own = MOwn<kCH, kBT>;              // C x kCH results
  constexpr int T64 = Own::TPW;
  constexpr int NB = X::NB;
  constexpr int SV = DV + 1, SC = kCH + 1;  // padded LDS rows
  constexpr int NSEG = kBT / kCH, LSEG = C / NSEG;
  // the direct-term products stream their left operands from global memory:
  // seven K-slices of prefetch where K allows
  constexpr int PFD = DV % 128 == 0 ? 7 : 3;
  constexpr int kB = kCH * SV > 3 * C * SC ? kCH * SV : 3 * C * SC;
  static_assert(kB >= C * SC + NSEG * kCH, "room for the cumulative sum");
  __shared__ double s_b[kB];              // staged right operands | dGamma
  __shared__ double s_P[C * (C + 1)], s_DA[C * (C + 1)];   // dP and beta dA, padded rows
  __shared__ double s_beta[C], s_dbp[2][C], s_kd[2][C], s_qd[2][C];
  __shared__ double s_fk[C], s_fq[C];
  __shared__ double s_red[4][kCH], s_red2[kCH], s_dGn[kCH];
  __shared__ double s_rm[kCH], s_sig[kCH];
  __shared__ int s_fb[kCH];

  const unsigned wg = blockIdx.x;
  const int t = threadIdx.x;
  const int blk = (int)((wg >> 3) % NB);
  const size_t chx = (size_t)((wg >> 3) / NB) * 8 + (wg & 7);
  if (chx >= n_ch) return;
  const int cflat = (int)(chx / H), h = (int)(chx % H);
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
  double *scr = scratch + ch * X::SIZE;
  const int cb = blk * kCH;

  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };   // token-head row
  // four consecutive columns of d_o per load
  auto dO_at = quad([&](int m, int c) {
    return m < nt ? ld4f(dO + row(m) * DV + c) : d4{0.0, 0.0, 0.0, 0.0};
  });
  auto khat = [&](int i, int c) {
    return i < nt ? (double)to_f32(k[row(i) * DK + c]) * s_fk[i] : 0.0;
  };
  auto qhat = [&](int i, int c) {
    return i < nt ? (double)to_f32(q[row(i) * DK + c]) * s_fq[i] : 0.0;
  };

  if (t < C) {
    s_beta[t] = t < nt ? (double)beta[row(t)] : 0.0;
    s_fk[t] = scr[X::FK + t];
    s_fq[t] = scr[X::FQ + t];
    s_dbp[0][t] = s_dbp[1][t] = s_kd[0][t] = s_kd[1][t] = s_qd[0][t] = s_qd[1][t] = 0.0;
  }
  const bool fbc = t < kCH && scr[X::FB + cb + t] != 0.0;
  if (t < kCH) {
    s_fb[t] = fbc;
    s_rm[t] = scr[X::RM + cb + t];
    s_sig[t] = scr[X::SIG + cb + t];
  }
  // the gate factors of (token i, channel cb + cl) from e (exact-path
  // channels: exp2 of G directly)
  const int8_t *sgn8 = reinterpret_cast<const int8_t *>(scr + X::SGN);
  auto gam_of = [&](double e, int i, int cl) {
    return s_fb[cl] ? sgn8[i * DK + cb + cl] * exp2(e) : ldexp(e, (int)s_rm[cl]);
  };
  auto khr_of = [&](double e, int i, int cl) {
    if (!s_fb[cl]) return s_sig[cl] / e;
    const double en = scr[X::E + (C - 1) * DK + cb + cl];
    return sgn8[i * DK + cb + cl] * sgn8[(C - 1) * DK + cb + cl] * exp2(en - e);
  };
  // the left operands of the direct-term products stream from global memory:
  // each product's first slices are issued ahead of the work before it
  auto fa_dx = quad([&](int m, int kk) { return ld4d(scr + X::DX + m * DV + kk); });
  auto fa_u = quad([&](int m, int kk) { return ld4d(Uc + m * DV + kk); });
  ARing<PFD> ring;
  mgemm_start(dO_at, ring);
  // S^T of this block, and dP and beta dA for the pair terms, into LDS (the
  // barrier also covers the per-token values above)
  for (int p = t; p < kCH * DV; p += kBT) s_b[(p / DV) * SV + p % DV] = Sc[cb * DV + p];
  for (int p = t; p < C * C; p += kBT) {
    s_P[(p / C) * (C + 1) + p % C] = scr[X::DP + p];
    s_DA[(p / C) * (C + 1) + p % C] = scr[X::DA + p];
  }
  const int anyfb = __syncthreads_or(fbc);

  double aq[T64][4], ak[T64][4], ag[T64][4];
  // this thread's raw split factors and normalised keys and queries, loaded
  // once: gamma Q, gamma K and K gamma_n / gamma follow from them
  double er[T64][4], kh[T64][4], qh[T64][4];
  float gseg[LSEG];
  d4 acc[T64];
  // dQT = dO S^T: dq = gamma dQT; dGamma = q gamma dQT.  M5 = dX S^T:
  // d(gamma K) = -Diag(beta) M5.
  {
    auto st = [&](int kk, int nn) { return s_b[nn * SV + kk]; };   // S^T (this block)
    // the epilogue's per-element factors are loaded before the product
    double gam[T64][4];
#pragma unroll
    for (int jj = 0; jj < T64; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = Own::row(r), c = cb + Own::col(jj);
        er[jj][r] = scr[X::E + i * DK + c];
        kh[jj][r] = khat(i, c);
        qh[jj][r] = qhat(i, c);
      }
    mgemm_run<kCH, DV, kBT, PFD>(dO_at, st, ring, acc);
    mgemm_start(fa_dx, ring);
#pragma unroll
    for (int jj = 0; jj < T64; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gam[jj][r] = gam_of(er[jj][r], Own::row(r), Own::col(jj));
        aq[jj][r] = gam[jj][r] * acc[jj][r];
        ag[jj][r] = gam[jj][r] * qh[jj][r] * acc[jj][r];
      }
    mgemm_run<kCH, DV, kBT, PFD>(fa_dx, st, ring, acc);
    mgemm_start(fa_u, ring);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = Own::row(r);
      double part = 0.0;
#pragma unroll
      for (int jj = 0; jj < T64; ++jj) {
        const double gk = gam[jj][r] * kh[jj][r];
        ak[jj][r] = -s_beta[i] * gam[jj][r] * acc[jj][r];
        ag[jj][r] -= s_beta[i] * gk * acc[jj][r];
        part -= gk * acc[jj][r];
      }
      add_row(s_dbp, i, part);
    }
  }
  __syncthreads();
  // dKH = U dS'^T: dk += (gamma_n / gamma) dKH; dGamma_i -= k (gamma_n/gamma) dKH,
  // and the same amount, summed over i, goes to dGamma_n.
  for (int p = t; p < kCH * DV; p += kBT) s_b[(p / DV) * SV + p % DV] = dSe[cb * DV + p];
  __syncthreads();
  // sum_j dS'[c][j] S[c][j] per channel of the block: 16 lanes per channel
  {
    static_assert(kCH * 16 == kBT, "16 threads per channel");
    const int cl = t >> 4, jp = t & 15;
    double sdot = 0.0;
#pragma unroll 8
    for (int j = jp; j < DV; j += 16) sdot += s_b[cl * SV + j] * Sc[(cb + cl) * DV + j];
    sdot = sum16(sdot);
    if (jp == 0) s_red2[cl] = sdot;
  }
  // the pair-term staging's inputs, in flight during this product
  constexpr int NST = C * kCH / kBT;
  double pe[NST];
  float pk[NST], pq[NST];
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int p = t + u * kBT, i = p / kCH, c = cb + p % kCH;
    pe[u] = scr[X::E + i * DK + c];
    pk[u] = i < nt ? to_f32(k[row(i) * DK + c]) : 0.f;
    pq[u] = i < nt ? to_f32(q[row(i) * DK + c]) : 0.f;
  }
  mgemm_run<kCH, DV, kBT, PFD>(fa_u, [&](int kk, int nn) { return s_b[nn * SV + kk]; }, ring,
                               acc);
#pragma unroll
  for (int jj = 0; jj < T64; ++jj) {
    const int cl = Own::col(jj);
    double col = 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double kr = khr_of(er[jj][r], Own::row(r), cl);
      const double term = kh[jj][r] * kr * acc[jj][r];
      ak[jj][r] += kr * acc[jj][r];
      ag[jj][r] -= term;
      col += term;
    }
    col += __shfl_xor(col, 16);
    col += __shfl_xor(col, 32);
    if ((t & 63) < 16) s_red[(t >> 6) & 3][cl] = col;
  }
  __syncthreads();
  if (t < kCH)
    s_dGn[t] = ((s_red[0][t] + s_red[1][t]) + (s_red[2][t] + s_red[3][t])) +
               rec[R::GN + cb + t] * s_red2[t];

  // ---- the pair terms: right operands F o K, E o K, E o Q of this block
  double *sFK = s_b, *sEK = s_b + C * SC, *sEQ = s_b + 2 * C * SC;
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int p = t + u * kBT, i = p / kCH, cl = p % kCH;
    const double e = s_fb[cl] ? 0.0 : pe[u];
    const double f = s_fb[cl] ? 0.0 : 1.0 / e;
    const double kh = (double)pk[u] * s_fk[i], qh = (double)pq[u] * s_fq[i];
    sFK[i * SC + cl] = f * kh;
    sEK[i * SC + cl] = e * kh;
    sEQ[i * SC + cl] = e * qh;
  }
  if (anyfb) {
    // channels too wide for the split: the four pair terms with exp2 per pair
    // (E holds G on these channels)
    auto sgn = [&](int i, int c) { return (double)sgn8[i * DK + c]; };
    for (int cg = 0; cg < kCH; cg += kBT / C) {
      const int c = cb + cg + t / C, i = t % C;
      if (!s_fb[c - cb]) continue;
      const double Gi = scr[X::E + i * DK + c], si = sgn(i, c);
      double R1 = 0.0, R2 = 0.0, C1 = 0.0, C2 = 0.0;
      for (int j = 0; j <= i; ++j) {
        const double r = si * sgn(j, c) * exp2(Gi - scr[X::E + j * DK + c]);
        const double kr = khat(j, c) * r;
        R1 = fma(s_P[i * (C + 1) + j], kr, R1);
        R2 = fma(s_DA[i * (C + 1) + j], kr, R2);
      }
      for (int m = i; m < C; ++m) {
        const double r = si * sgn(m, c) * exp2(scr[X::E + m * DK + c] - Gi);
        C1 = fma(s_DA[m * (C + 1) + i], khat(m, c) * r, C1);
        C2 = fma(s_P[m * (C + 1) + i], qhat(m, c) * r, C2);
      }
      scr[X::AQ + i * DK + c] = R1;
      scr[X::AK + i * DK + c] = R2;
      scr[X::X3 + i * DK + c] = C1;
      scr[X::X4 + i * DK + c] = C2;
    }
    __threadfence_block();
  }
  __syncthreads();
  {
    // the split factor of each owned (token, channel): e for the R terms,
    // then f for the C terms (0 on exact-path channels)
    double ef[T64][4];
    auto split = [&](bool want_f) {
#pragma unroll
      for (int jj = 0; jj < T64; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double e = er[jj][r];
          ef[jj][r] = s_fb[Own::col(jj)] ? 0.0 : want_f ? 1.0 / e : e;
        }
    };
    split(false);
    // the gates of this thread's dalpha segment, in flight during the products
#pragma unroll
    for (int u = 0; u < LSEG; ++u) {
      const int i = LSEG * (t / kCH) + u;
      gseg[u] = i < nt ? g[row(i) * DK + cb + t % kCH] : 1.f;
    }
    // R1 = E o (dP (F o K)): into dq and dGamma (+ q R1); dq is then complete
    mgemm<kCH, C, kBT, 1>([&](int m, int kk) { return s_P[m * (C + 1) + kk]; },
                       [&](int kk, int nn) { return sFK[kk * SC + nn]; }, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = Own::row(r);
      double dqd = 0.0;
#pragma unroll
      for (int jj = 0; jj < T64; ++jj) {
        const int cl = Own::col(jj), c = cb + cl;
        double R1 = ef[jj][r] * acc[jj][r];
        if (s_fb[cl]) R1 = scr[X::AQ + i * DK + c];      // exact-path channel
        const double gq = aq[jj][r] + R1;
        ag[jj][r] += qh[jj][r] * R1;
        if (l2norm) {
          // the gradient with respect to the normalised row; the
          // normalisation's Jacobian is applied once every channel is done
          scr[X::AQ + i * DK + c] = gq;
          dqd += qh[jj][r] * gq;
        } else if (i < nt) {
          dq[row(i) * DK + c] = (float)gq;
        }
      }
      if (l2norm) add_row(s_qd, i, dqd);
    }
    // R2 = E o ((beta dA) (F o K)): into dk and dGamma (+ k R2)
    mgemm<kCH, C, kBT, 1>([&](int m, int kk) { return s_DA[m * (C + 1) + kk]; },
                       [&](int kk, int nn) { return sFK[kk * SC + nn]; }, acc);
#pragma unroll
    for (int jj = 0; jj < T64; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double R2 = ef[jj][r] * acc[jj][r];
        ak[jj][r] += R2;
        ag[jj][r] += kh[jj][r] * R2;
      }
    split(true);
    // C1 = F o ((beta dA)^T (E o K)): into dk and dGamma (- k C1)
    mgemm<kCH, C, kBT, 1>([&](int m, int kk) { return s_DA[kk * (C + 1) + m]; },
                       [&](int kk, int nn) { return sEK[kk * SC + nn]; }, acc);
#pragma unroll
    for (int jj = 0; jj < T64; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double C1 = ef[jj][r] * acc[jj][r];
        ak[jj][r] += C1;
        ag[jj][r] -= kh[jj][r] * C1;
      }
    // C2 = F o (dP^T (E o Q)): into dk and dGamma (- k C2)
    mgemm<kCH, C, kBT, 1>([&](int m, int kk) { return s_P[kk * (C + 1) + m]; },
                       [&](int kk, int nn) { return sEQ[kk * SC + nn]; }, acc);
    // exact-path channels, the last token's dGamma_n, and dk
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = Own::row(r);
      double dkd = 0.0;
#pragma unroll
      for (int jj = 0; jj < T64; ++jj) {
        const int cl = Own::col(jj), c = cb + cl;
        const double C2 = ef[jj][r] * acc[jj][r];
        ak[jj][r] += C2;
        ag[jj][r] -= kh[jj][r] * C2;
        if (s_fb[cl]) {
          const double R2 = scr[X::AK + i * DK + c];
          const double C1 = scr[X::X3 + i * DK + c], C2x = scr[X::X4 + i * DK + c];
          ak[jj][r] += R2 + C1 + C2x;
          ag[jj][r] += kh[jj][r] * (R2 - C1 - C2x);
        }
        if (i == C - 1) ag[jj][r] += s_dGn[cl];
        if (l2norm) {
          scr[X::AK + i * DK + c] = ak[jj][r];
          dkd += kh[jj][r] * ak[jj][r];
        } else if (i < nt) {
          dk[row(i) * DK + c] = (float)ak[jj][r];
        }
      }
      if (l2norm) add_row(s_kd, i, dkd);
    }
  }
  __syncthreads();                      // every read of the staged operands done
  // dln|alpha_s| = sum_{i >= s} dGamma_i; dalpha = dln|alpha| / alpha.
  // NSEG segments of C / NSEG tokens per channel, then the segment offsets.
  double *s_ag = s_b, *s_seg = s_b + C * SC;
#pragma unroll
  for (int jj = 0; jj < T64; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_ag[Own::row(r) * SC + Own::col(jj)] = ag[jj][r];
  __syncthreads();
  {
    const int cl = t % kCH, sgm = t / kCH;
    double sum = 0.0;
#pragma unroll
    for (int i = LSEG * sgm; i < LSEG * sgm + LSEG; ++i) sum += s_ag[i * SC + cl];
    s_seg[sgm * kCH + cl] = sum;
    __syncthreads();
    double acc2 = 0.0;
    for (int s2 = NSEG - 1; s2 > sgm; --s2) acc2 += s_seg[s2 * kCH + cl];
    const double floor_mag = exp2(kLog2Floor);
#pragma unroll
    for (int i = LSEG * sgm + LSEG - 1; i >= LSEG * sgm; --i) {
      acc2 += s_ag[i * SC + cl];
      if (i < nt) {
        const double a = gseg[i - LSEG * sgm];
        const double am = fabs(a) < floor_mag ? (a < 0.0 ? -floor_mag : floor_mag) : a;
        dg[row(i) * DK + cb + cl] = (float)(acc2 / am);
      }
    }
  }
  // this block's parts of dbeta and of the normalisation dots
  if (t < C) {
    scr[X::DB + (1 + blk) * C + t] = s_dbp[0][t] + s_dbp[1][t];
    scr[X::QD + blk * C + t] = s_qd[0][t] + s_qd[1][t];
    scr[X::KD + blk * C + t] = s_kd[0][t] + s_kd[1][t];
  }
}

// --------------------------------------------------------------------------
// dbeta (the prep kernel's part plus every channel block's, in a fixed
// order) and, with q/k normalisation, dx = f_x (dxhat - xhat (xhat . dxhat)).
constexpr int kFT = 256;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kFT) void f64_bwd_final(
    const TIn *__restrict__ q, const TIn *__restrict__ k, int H, int N, SeqTable tab,
    const double *__restrict__ scratch, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dbeta, int l2norm) {
  using X = Scr<DK, DV>;
  constexpr int NB = X::NB;
  __shared__ double s_qd[C], s_kd[C], s_fq[C], s_fk[C];
  const int cflat = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (cflat >= tab.chunk_off[N]) return;
  const int n = find_seq(tab.chunk_off, N, cflat);
  const int lc = cflat - tab.chunk_off[n];
  const int t0 = tab.seq_start[n] + lc * C;
  const int nt = min(C, tab.seq_len[n] - lc * C);
  const double *scr = scratch + ((size_t)cflat * H + h) * X::SIZE;
  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };
  if (t < nt) {
    double db = 0.0, qd = 0.0, kd = 0.0;
#pragma unroll
    for (int b = 0; b <= NB; ++b) db += scr[X::DB + b * C + t];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      qd += scr[X::QD + b * C + t];
      kd += scr[X::KD + b * C + t];
    }
    dbeta[row(t)] = (float)db;
    s_qd[t] = qd;
    s_kd[t] = kd;
    s_fq[t] = scr[X::FQ + t];
    s_fk[t] = scr[X::FK + t];
  }
  if (!l2norm) return;                  // uniform across the block
  __syncthreads();
#pragma unroll 4
  for (int p = t; p < nt * DK; p += kFT) {
    const int i = p / DK, c = p % DK;
    const double qh = to_f32(q[row(i) * DK + c]) * s_fq[i];
    const double kh = to_f32(k[row(i) * DK + c]) * s_fk[i];
    dq[row(i) * DK + c] = (float)(s_fq[i] * (scr[X::AQ + p] - qh * s_qd[i]));
    dk[row(i) * DK + c] = (float)(s_fk[i] * (scr[X::AK + p] - kh * s_kd[i]));
  }
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
  const TIn *tq = static_cast<const TIn *>(q), *tk = static_cast<const TIn *>(k);
  hipLaunchKernelGGL((f64_bwd_state<DK, DV>), dim3(xcd_grid(DV / kBV, N * H)), dim3(kThreads), 0,
                     stream,
                     dO, dS_T, H, N, tab, records, rec_doubles, dU_chunks, dSe_chunks, dS0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_chunks_ub == 0) return e;
  hipLaunchKernelGGL((f64_bwd_prep<TIn, DK, DV>), dim3((unsigned)n_chunks_ub, H), dim3(kBT), 0,
                     stream, tq, tk, static_cast<const TIn *>(v), g, beta, dO, H, N, tab,
                     records, rec_doubles, U_chunks, dU_chunks, scratch, dv, signed_gates, l2norm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (channel block, chunk, head) workgroups, eight chunk-heads per XCD round
  const size_t n_ch = n_chunks_ub * (size_t)H;
  const size_t n_wg = (n_ch + 7) / 8 * 8 * (DK / kCH);
  hipLaunchKernelGGL((f64_bwd_pairs<TIn, DK, DV>), dim3((unsigned)n_wg), dim3(kBT), 0, stream,
                     tq, tk, g, beta, dO, H, N, tab, records, rec_doubles, S_chunks, U_chunks,
                     dSe_chunks, scratch, n_ch, dq, dk, dg, l2norm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((f64_bwd_final<TIn, DK, DV>), dim3((unsigned)n_chunks_ub, H), dim3(kFT), 0,
                     stream, tq, tk, H, N, tab, scratch, dq, dk, dbeta, l2norm);
  return hipGetLastError();
}

}  // namespace

size_t f64_bwd_scratch_bytes(int dk, int dv) {
  const size_t nb = (size_t)dk / kCH;
  return sizeof(double) * ((size_t)C * dv + 5 * (size_t)C * dk + 2 * (size_t)C * C + 3 * dk +
                           2 * (size_t)C + (1 + 3 * nb) * (size_t)C + (size_t)C * dk / 8);
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
