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
//   f64_intra  grid (chunks, heads): G, pi, then A and P as sums over the
//              channels of per-pair ratio products (each ratio is one product
//              of two factors taken about the channel's midpoint, or exp2 of
//              the difference where the channel spans too many binary orders),
//              T blockwise (diagonal 16 x 16 blocks by forward substitution,
//              then block rows), then W, Ubar, gamma*Q, K_hat, gamma_n.
//              T and A / beta stay in the record for the backward pass.
//   f64_inter  grid (dv blocks x sequences x heads): the serial chunk loop on
//              an fp64 state slice held in LDS, each product an LDS-staged
//              block product; for the backward pass it can also keep the
//              state entering each chunk and the chunk's U.
// This path favours clarity and fp64 accuracy (fp32 inputs carry a 1e-5
// relative tolerance) over speed; bf16 inputs use the matrix-core path.
#include "f64_common.h"

namespace ckda {
namespace {

using namespace f64;

constexpr int kCB = 32;              // channels per block of the A and P products

// The record kernel runs 512 threads (two waves per SIMD over one block's LDS).
constexpr int kIT = 512;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kIT) void f64_intra(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, int H, int N, SeqTable tab,
    double *__restrict__ records, size_t rec_doubles, int signed_gates, int l2norm) {
  using R = Rec<DK, DV>;
  constexpr int kU = 3 * C * (kCB + 1);  // the A/P product operands of one channel block
  static_assert(kU >= 3 * 256, "room for the blocked inverse's partial products");
  __shared__ double s_G[C * DK > C * (C + 1) ? C * DK : C * (C + 1)];  // gate factors, later T
  __shared__ uint8_t s_par[C * DK];
  __shared__ double s_A[C * (C + 1)];
  __shared__ double s_u[kU];            // A/P operands | blocked-inverse partial products
  __shared__ double s_beta[C], s_fk[C], s_fq[C];
  __shared__ double s_R[DK], s_sig[DK];
  __shared__ int s_fb[DK];
  __shared__ int s_anyfb;

  const int cflat = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (cflat >= tab.chunk_off[N]) return;
  if (t == 0) s_anyfb = 0;
  const int n = find_seq(tab.chunk_off, N, cflat);
  const int lc = cflat - tab.chunk_off[n];
  const int t0 = tab.seq_start[n] + lc * C;
  const int nt = min(C, tab.seq_len[n] - lc * C);
  double *rec = records + ((size_t)cflat * H + h) * rec_doubles;

  auto row = [&](int i) { return (size_t)(t0 + i) * H + h; };   // token-head row

  // Every input of the chunk is loaded up front, four consecutive channels
  // per load, so a workgroup waits for global memory once.  The values are
  // staged in LDS as fp32 just before the Ubar product.
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f), one4 = make_float4(1.f, 1.f, 1.f, 1.f);
  constexpr int NVL = C * DV / (4 * kIT);
  float4 vpre[NVL];
#pragma unroll
  for (int u = 0; u < NVL; ++u) {
    const int e = 4 * (t + u * kIT), i = e / DV;
    vpre[u] = i < nt ? load4_f32(v + row(i) * DV + e % DV) : zero4;
  }
  // the gates
  constexpr int NGL = C * DK / (4 * kIT);
  float4 gpre[NGL];
#pragma unroll
  for (int u = 0; u < NGL; ++u) {
    const int e = 4 * (t + u * kIT), i = e / DK;
    gpre[u] = i < nt ? *reinterpret_cast<const float4 *>(g + row(i) * DK + e % DK) : one4;
  }
  // the keys and queries of every kCB-channel block of the A/P products: in
  // block b, thread t takes token t / (kCB / 4) and channels
  // b kCB + 4 (t % (kCB / 4)) .. + 3
  constexpr int NKB = DK / kCB;
  static_assert(C * kCB == 4 * kIT, "one load of four channels per thread and block");
  float4 rk[NKB], rq[NKB];
  const int ki = t / (kCB / 4), kc = 4 * (t % (kCB / 4));
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
    rk[b] = ki < nt ? load4_f32(k + row(ki) * DK + b * kCB + kc) : zero4;
    rq[b] = ki < nt ? load4_f32(q + row(ki) * DK + b * kCB + kc) : zero4;
  }

  // ---- gates: |alpha| (floored at 2^kLog2Floor, so that a zero gate keeps
  // the products finite) and the sign of every (token, channel) in parallel,
  // then per channel the inclusive scans: the running product of the
  // magnitudes and the parity of the negatives.
#pragma unroll
  for (int u = 0; u < NGL; ++u)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int p = 4 * (t + u * kIT) + cc;
      const float a = cc == 0 ? gpre[u].x : cc == 1 ? gpre[u].y : cc == 2 ? gpre[u].z : gpre[u].w;
      s_G[p] = fmax(fabs((double)a), ldexp(1.0, (int)kLog2Floor));
      s_par[p] = (uint8_t)(signed_gates && a < 0.f);   // KDA mode: signs ignored
    }
  __syncthreads();
  {
    // gamma_i = prod_{s<=i} |alpha_s| is carried as m 2^x with m in [0.5, 1),
    // renormalised after every factor, so no product leaves fp64's range and
    // G = log2 gamma (x - 1 <= G < x) is never needed for the usual channel.
    // Each channel's tokens are cut into NSG segments, one thread each: a pass
    // over the segment from 1, the segments' totals combined in order, then a
    // second pass from the segment's prefix.  Combining: (m1, x1) (m2, x2) =
    // (m, x1 + x2 + d) with m 2^d = m1 m2.
    constexpr int NSG = kIT / DK, LS = C / NSG;
    static_assert(NSG * DK == kIT && NSG * LS == C, "segments of the gate scan");
    const int c = t % DK, sg = t / DK, i0 = sg * LS;
    double *tot_m = s_u, *tot_x = s_u + kIT, *tot_hi = s_u + 2 * kIT, *tot_lo = s_u + 3 * kIT,
           *tot_p = s_u + 4 * kIT;       // per (segment, channel); s_u is free until A and P
    static_assert(5 * kIT <= kU, "room for the segment totals");
    double m = 0.5;
    int x = 1, xhi = 1, xlo = 1;
    uint8_t par = 0;
#pragma unroll
    for (int i = i0; i < i0 + LS; ++i) {
      int dx;
      m = frexp(m * s_G[i * DK + c], &dx);
      x += dx;
      xhi = max(xhi, x);
      xlo = min(xlo, x);
      par ^= s_par[i * DK + c];
      s_par[i * DK + c] = par;            // parity within the segment, for now
    }
    tot_m[t] = m;
    tot_x[t] = x;
    tot_hi[t] = xhi;
    tot_lo[t] = xlo;
    tot_p[t] = par;
    __syncthreads();
    // this segment's prefix, and bounds on the channel's G: a token of segment
    // s2 has x in [xp + x_local - 1, xp + x_local], so lo <= G < hi (the chunk
    // start, G = 0, counts)
    double mp = 0.5, mseg = 0.5;
    int xp = 1, xseg = 1, hi = 1, lo = 0;
    uint8_t pp = 0, pseg = 0;
    for (int s2 = 0; s2 < NSG; ++s2) {
      const int u = s2 * DK + c;
      if (s2 == sg) {
        mseg = mp;
        xseg = xp;
        pseg = pp;
      }
      hi = max(hi, xp + (int)tot_hi[u]);
      lo = min(lo, xp + (int)tot_lo[u] - 2);
      int dx;
      mp = frexp(mp * tot_m[u], &dx);
      xp += (int)tot_x[u] + dx;
      pp ^= (uint8_t)tot_p[u];
    }
    // Pair ratios are formed as e_i f_j with e = 2^(G - Rm), f = 1 / e about
    // an integer midpoint Rm of the channel's range (gamma = e 2^Rm is then an
    // exact scaling of e).  Past +-1000 binary orders e f could leave fp64's
    // range; such a channel keeps G itself and takes exp2 per pair.
    const int Rm = (hi + lo) / 2;
    const bool fb = hi - lo > 2000;
    m = mseg;
    x = xseg;
#pragma unroll
    for (int i = i0; i < i0 + LS; ++i) {     // the same products again, now scaled
      int dx;
      m = frexp(m * s_G[i * DK + c], &dx);
      x += dx;
      s_G[i * DK + c] = fb ? (double)x + log2(m) : ldexp(m, x - Rm);   // G, or |e| = 2^(G - Rm)
      s_par[i * DK + c] ^= pseg;
    }
    if (sg == NSG - 1)     // sign(gamma_n) 2^(G_n - Rm)
      s_sig[c] = fb ? 0.0 : ((par ^ pseg) ? -1.0 : 1.0) * ldexp(m, x - Rm);
    if (sg == 0) {
      s_R[c] = (double)Rm;
      s_fb[c] = fb;
      if (fb) s_anyfb = 1;
    }
  }
  // ---- optional L2 normalisation of q and k per token: (sum x^2 + 1e-6)^(-1/2)
  if (t < C) {
    double fk = 1.0, fq = 1.0;
    if (l2norm && t < nt) {
      double sk = 1e-6, sq = 1e-6;
      for (int c = 0; c < DK; ++c) {
        const double kk = to_f32(k[row(t) * DK + c]), qq = to_f32(q[row(t) * DK + c]);
        sk += kk * kk;
        sq += qq * qq;
      }
      fk = 1.0 / sqrt(sk);
      fq = 1.0 / sqrt(sq);
    }
    s_fk[t] = fk;
    s_fq[t] = fq;
    s_beta[t] = t < nt ? (double)beta[row(t)] : 0.0;
  }
  __syncthreads();

  // ---- A (strictly lower) and P (lower incl. diagonal) on the fp64 matrix
  // cores.  With the ratio split r_ij = e_i f_j about each channel's midpoint,
  // A/beta = (K o E)(K o F)^T and P = (Q o E)(K o F)^T (K, Q the normalised
  // keys and queries), summed over blocks of kCB channels staged in LDS.
  // Channels too wide for the split are left out of the products (e = f = 0)
  // and added pair by pair afterwards.
  {
    using Own = MOwn<C, kIT>;
    constexpr int TP = Own::TPW, SB = kCB + 1;
    double *sKE = s_u, *sQE = s_u + C * SB, *sKF = s_u + 2 * C * SB;
    d4 accA[TP], accP[TP];
#pragma unroll
    for (int jj = 0; jj < TP; ++jj) accA[jj] = accP[jj] = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
    for (int c0 = 0; c0 < DK; c0 += kCB) {
      __syncthreads();                  // the previous block's products are done
      // the split factors, and the gamma-scaled records of this thread's four
      // (token, channel) pairs: gamma Q, gamma K, K gamma_n / gamma and
      // gamma_n (masked tokens have k = q = 0)
      const int i = ki;
      d4 oq, ok, okh;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cl = kc + u, c = c0 + cl;
        const float rku = u == 0 ? rk[0].x : u == 1 ? rk[0].y : u == 2 ? rk[0].z : rk[0].w;
        const float rqu = u == 0 ? rq[0].x : u == 1 ? rq[0].y : u == 2 ? rq[0].z : rq[0].w;
        const double G = s_G[i * DK + c], sg = s_par[i * DK + c] ? -1.0 : 1.0;
        const double kh = (double)rku * s_fk[i], qh = (double)rqu * s_fq[i];
        double e = 0.0, f = 0.0, gam, khr;
        if (!s_fb[c]) {
          const double eu = G;           // |e| = 2^(G - Rm) for such a channel
          e = sg * eu;
          f = sg / eu;
          gam = sg * ldexp(eu, (int)s_R[c]);
          khr = s_sig[c] * f;
        } else {
          const double Gn = s_G[(C - 1) * DK + c];
          const double sn = s_par[(C - 1) * DK + c] ? -1.0 : 1.0;
          gam = sg * exp2(G);
          khr = sg * sn * exp2(Gn - G);
        }
        oq[u] = qh * gam;
        ok[u] = kh * gam;
        okh[u] = kh * khr;
        if (i == C - 1) rec[R::GN + c] = gam;
        sKE[i * SB + cl] = kh * e;
        sQE[i * SB + cl] = qh * e;
        sKF[i * SB + cl] = kh * f;
      }
      *reinterpret_cast<d4 *>(rec + R::QT + i * DK + c0 + kc) = oq;
      *reinterpret_cast<d4 *>(rec + R::GK + i * DK + c0 + kc) = ok;
      *reinterpret_cast<d4 *>(rec + R::KH + i * DK + c0 + kc) = okh;
      __syncthreads();
#pragma unroll
      for (int b = 0; b + 1 < NKB; ++b) {   // the next block's keys and queries move up
        rk[b] = rk[b + 1];
        rq[b] = rq[b + 1];
      }
      auto kf = [&](int kk, int nn) { return sKF[nn * SB + kk]; };   // (K o F)^T
      mgemm<C, kCB, kIT, 1, false>([&](int m, int kk) { return sKE[m * SB + kk]; }, kf, accA);
      mgemm<C, kCB, kIT, 1, false>([&](int m, int kk) { return sQE[m * SB + kk]; }, kf, accP);
    }
    if (s_anyfb) {
      // r_ij = sign_i sign_j 2^(G_i - G_j) one pair at a time (j <= i)
      for (int c = 0; c < DK; ++c) {
        if (!s_fb[c]) continue;         // uniform across the block
#pragma unroll
        for (int jj = 0; jj < TP; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = Own::row(r), j = Own::col(jj);
            if (j > i || i >= nt) continue;
            const double sgn = (s_par[i * DK + c] ^ s_par[j * DK + c]) ? -1.0 : 1.0;
            const double rr = sgn * exp2(s_G[i * DK + c] - s_G[j * DK + c]);
            const double kj = (double)to_f32(k[row(j) * DK + c]) * s_fk[j] * rr;
            accA[jj][r] += (double)to_f32(k[row(i) * DK + c]) * s_fk[i] * kj;
            accP[jj][r] += (double)to_f32(q[row(i) * DK + c]) * s_fq[i] * kj;
          }
      }
    }
#pragma unroll
    for (int jj = 0; jj < TP; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = Own::row(r), j = Own::col(jj);
        const double a = j < i ? accA[jj][r] : 0.0;
        s_A[i * (C + 1) + j] = s_beta[i] * a;
        rec[R::AH + i * C + j] = a;
        rec[R::P + i * C + j] = j <= i ? accP[jj][r] : 0.0;
      }
  }

  __threadfence_block();   // scratch is read back by this workgroup only
  __syncthreads();

  // ---- T = (I + A)^-1, blockwise over 16 x 16 blocks: the four diagonal
  // blocks by forward substitution (one column per thread, held in
  // registers), then block rows I = 1..3 in turn on the fp64 matrix cores:
  // T_IJ = -T_II M_IJ with M_IJ = sum_{J<=K<I} A_IK T_KJ, one wave per J < I.
  double *s_T = s_G;     // G is dead; T is C x (C+1)
  for (int p = t; p < C * (C + 1); p += kIT) s_T[p] = (p / (C + 1) == p % (C + 1)) ? 1.0 : 0.0;
  __syncthreads();
  if (t < C) {
    // column jl of diagonal block I: x_r = -sum_{m<r} A_rm x_m below the unit entry
    const int I = t >> 4, jl = t & 15;
    const double *a = s_A + 16 * I * (C + 1) + 16 * I;
    double x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      double acc = 0.0;
#pragma unroll
      for (int m = 0; m < r; ++m) acc = fma(a[r * (C + 1) + m], x[m], acc);
      x[r] = r < jl ? 0.0 : r == jl ? 1.0 : -acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s_T[(16 * I + r) * (C + 1) + 16 * I + jl] = x[r];
  }
  __syncthreads();
  {
    // operand layout of the fp64 product (lane l, K-slice sl of 4):
    // A(l % 16, 4 sl + l / 16), B(4 sl + l / 16, l % 16); accumulator entry r
    // holds (4 r + l / 16, l % 16), so M's K-slice sl is the lane's entry sl
    const int w = t >> 6, l = t & 63, lr = l & 15, lk = l >> 4;
    for (int I = 1; I < C / 16; ++I) {
      if (w < I) {
        const int J = w;
        d4 m4 = {0.0, 0.0, 0.0, 0.0};
        for (int K = J; K < I; ++K)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            m4 = __builtin_amdgcn_mfma_f64_16x16x4f64(
                s_A[(16 * I + lr) * (C + 1) + 16 * K + 4 * sl + lk],
                s_T[(16 * K + 4 * sl + lk) * (C + 1) + 16 * J + lr], m4, 0, 0, 0);
        d4 t4 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          t4 = __builtin_amdgcn_mfma_f64_16x16x4f64(
              s_T[(16 * I + lr) * (C + 1) + 16 * I + 4 * sl + lk], m4[sl], t4, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_T[(16 * I + 4 * r + lk) * (C + 1) + 16 * J + lr] = -t4[r];
      }
      __syncthreads();
    }
  }

  // ---- T, W = T Diag(beta) (gamma*K), Ubar = T Diag(beta) V, formed
  // transposed on the fp64 matrix cores 64 columns at a time:
  // W^T = (gamma*K)^T (T Diag(beta))^T and Ubar^T = V^T (T Diag(beta))^T, the
  // left operand streamed from global memory, the right one read from T in LDS.
  for (int p = t; p < C * C; p += kIT) rec[R::TI + p] = s_T[(p % C) * (C + 1) + p / C];   // T^T
  {
    using Own = MOwn<C, kIT>;
    constexpr int TP = Own::TPW;
    auto tbt = [&](int kk, int nn) { return s_T[nn * (C + 1) + kk] * s_beta[kk]; };
    d4 acc[TP];
#pragma unroll 1
    for (int cb = 0; cb < DK; cb += 64) {
      mgemm<C, C, kIT>([&](int m, int kk) { return rec[R::GK + kk * DK + cb + m]; }, tbt, acc);
#pragma unroll
      for (int jj = 0; jj < TP; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rec[R::W + Own::col(jj) * DK + cb + Own::row(r)] = acc[jj][r];
    }
    float *s_v = reinterpret_cast<float *>(s_u);   // [C][DV + 1] (the A/P operands are done)
    static_assert(C * (DV + 1) <= 2 * kU, "room for V in fp32");
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int e = 4 * (t + u * kIT), i = e / DV, c = e % DV;
      s_v[i * (DV + 1) + c] = vpre[u].x;
      s_v[i * (DV + 1) + c + 1] = vpre[u].y;
      s_v[i * (DV + 1) + c + 2] = vpre[u].z;
      s_v[i * (DV + 1) + c + 3] = vpre[u].w;
    }
    __syncthreads();
#pragma unroll 1
    for (int cb = 0; cb < DV; cb += 64) {
      mgemm<C, C, kIT>([&](int m, int kk) { return (double)s_v[kk * (DV + 1) + cb + m]; }, tbt,
                       acc);
#pragma unroll
      for (int jj = 0; jj < TP; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          rec[R::UB + Own::col(jj) * DV + cb + Own::row(r)] = acc[jj][r];
    }
  }
}

// Serial pass over the chunks of one (sequence, head, BV-column block).  The
// products run on the fp64 matrix cores with their right operands (S, U) in
// LDS; three barriers per chunk order the phases.  BV is 32, or 16 when the
// 32-column grid would leave most of the GPU idle.
template <int DK, int DV, int BV>
__global__ __launch_bounds__(kThreads) void f64_inter(
    const float *S0, int H, int N, SeqTable tab, const double *__restrict__ records,
    size_t rec_doubles, void *__restrict__ o, float *S_T, int o_bf16,
    double *__restrict__ S_chunks, double *__restrict__ U_chunks) {
  using R = Rec<DK, DV>;
  using Own = MOwn<BV>;
  constexpr int TPW = Own::TPW;
  __shared__ double s_S[DK * BV];
  __shared__ double s_U[C * BV];

  constexpr int NV = DV / BV;
  const int t = threadIdx.x;
  int rh, jb;
  if (!xcd_block(NV, N * H, rh, jb)) return;
  const int n = tab.order[rh / H], h = rh % H;
  const int len = tab.seq_len[n], start = tab.seq_start[n];
  const int nch = (len + C - 1) / C;
  const size_t sbase = ((size_t)n * H + h) * DK * DV + (size_t)jb * BV;

  for (int p = t; p < DK * BV; p += kThreads) {
    const int c = p / BV, j = p % BV;
    s_S[p] = S0 ? (double)S0[sbase + (size_t)c * DV + j] : 0.0;
  }
  __syncthreads();

  for (int lc = 0; lc < nch; ++lc) {
    const size_t ch = (size_t)(tab.chunk_off[n] + lc) * H + h;
    const double *rec = records + ch * rec_doubles;
    const int nt = min(C, len - lc * C);
    // the left operands are records, independent of the state: the first
    // slices of each product are issued ahead of the work before it
    auto fa_w = [&](int m, int kk) { return rec[R::W + m * DK + kk]; };
    auto fa_o = [&](int m, int kk) {
      return kk < DK ? rec[R::QT + m * DK + kk] : rec[R::P + m * C + kk - DK];
    };
    auto fa_k = [&](int half) {
      return [&, half](int m, int kk) { return rec[R::KH + kk * DK + half * 64 + m]; };
    };
    ARing<> ring_w, ring_o, ring_k[DK / 64];
    mgemm_start(fa_w, ring_w);
    if (S_chunks)
      for (int p = t; p < DK * BV; p += kThreads)
        S_chunks[ch * DK * DV + (size_t)(p / BV) * DV + jb * BV + p % BV] = s_S[p];
    // U = Ubar - W S
    {
      d4 acc[TPW];
      double ub[TPW][4];                   // the epilogue's Ubar, loaded ahead
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ub[jj][r] = rec[R::UB + Own::row(r) * DV + jb * BV + Own::col(jj)];
      mgemm_run<BV, DK>(fa_w, [&](int kk, int nn) { return s_S[kk * BV + nn]; }, ring_w, acc);
      if (o)
        mgemm_start(fa_o, ring_o);
      else
        mgemm_start(fa_k(0), ring_k[0]);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = Own::row(r), j = Own::col(jj);
          const double u = ub[jj][r] - acc[jj][r];
          s_U[i * BV + j] = u;
          if (U_chunks) U_chunks[ch * C * DV + (size_t)i * DV + jb * BV + j] = u;
        }
    }
    __syncthreads();         // U complete
    // O = (gamma Q) S + P U, as one product over [S; U]
    if (o) {
      d4 acc[TPW];
      mgemm_run<BV, DK + C>(
          fa_o,
          [&](int kk, int nn) { return kk < DK ? s_S[kk * BV + nn] : s_U[(kk - DK) * BV + nn]; },
          ring_o, acc);
      mgemm_start(fa_k(0), ring_k[0]);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = Own::row(r), j = Own::col(jj);
          if (i >= nt) continue;
          const size_t oi = ((size_t)(start + lc * C + i) * H + h) * DV + jb * BV + j;
          if (o_bf16)
            static_cast<__hip_bfloat16 *>(o)[oi] = __float2bfloat16((float)acc[jj][r]);
          else
            static_cast<float *>(o)[oi] = (float)acc[jj][r];
        }
      __syncthreads();       // every read of S done before it is rewritten
    }
    // S' = Diag(gamma_n) S + K_hat^T U, 64 state rows at a time (in place: each
    // thread rewrites only its own elements, and the product reads U only)
#pragma unroll
    for (int half = 0; half < DK / 64; ++half) {
      d4 acc[TPW];
      double gn[4];                        // gamma_n of this thread's state rows
#pragma unroll
      for (int r = 0; r < 4; ++r) gn[r] = rec[R::GN + half * 64 + Own::row(r)];
      mgemm_run<BV, C>(fa_k(half), [&](int kk, int nn) { return s_U[kk * BV + nn]; },
                        ring_k[half], acc);
      if (half + 1 < DK / 64) mgemm_start(fa_k(half + 1), ring_k[half + 1]);
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = half * 64 + Own::row(r), j = Own::col(jj);
          s_S[c * BV + j] = gn[r] * s_S[c * BV + j] + acc[jj][r];
        }
    }
    __syncthreads();         // S' complete, U free
  }
  if (S_T)
    for (int p = t; p < DK * BV; p += kThreads) {
      const int c = p / BV, j = p % BV;
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
    hipLaunchKernelGGL((f64_intra<TIn, DK, DV>), dim3((unsigned)n_chunks_ub, H), dim3(kIT),
                       0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                       static_cast<const TIn *>(v), g, beta, H, N, tab,
                       static_cast<double *>(records), rec_doubles, signed_gates, l2norm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // fewer 32-column workgroups than compute units: 16-column blocks instead
  if ((size_t)(DV / kBV) * N * H < 256) {
    hipLaunchKernelGGL((f64_inter<DK, DV, kBV / 2>), dim3(xcd_grid(DV / (kBV / 2), N * H)),
                       dim3(kThreads), 0, stream, S0, H, N, tab,
                       static_cast<const double *>(records), rec_doubles, o, S_T, o_bf16,
                       S_chunks, U_chunks);
  } else {
    hipLaunchKernelGGL((f64_inter<DK, DV, kBV>), dim3(xcd_grid(DV / kBV, N * H)), dim3(kThreads), 0,
                       stream, S0, H, N, tab, static_cast<const double *>(records), rec_doubles,
                       o, S_T, o_bf16, S_chunks, U_chunks);
  }
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
