// Fused chunkwise CKDA forward for bf16 q/k/v on CDNA4 matrix cores.
//
// One workgroup owns one (sequence, head, 64-column block of dv) and walks the
// sequence's chunks of C = 64 tokens in order, keeping its slice of the fp32
// state (dk x 64) in MFMA accumulators for the whole sequence.  Each chunk is
// read from HBM once (the dv blocks of one head share q/k/alpha through the
// XCD's L2) and o is written once: the only HBM traffic is the compulsory one.
//
// Chunk algebra (update rule: blog post "One update, one quarter turn", ELI5
// "The mirror", unrolled over a chunk with incoming state S; r_ij is the gate
// product over tokens j < s <= i, gamma_i = r_i0):
//   A_ij = beta_i sum_c k_ic r_ij,c k_jc (i > j)    T = (I + A)^-1
//   X    = V - (gamma K) S                           U = T Diag(beta) X
//   O    = (gamma Q) S + P U,   P_ij = sum_c q_ic r_ij,c k_jc (j <= i)
//   S'   = Diag(gamma_n) S + (K gamma_n / gamma)^T U
//
// Signed gates (CKDA summary, "Methodology in Plain English": magnitudes live
// in log space, the sign apart): per channel the chunk keeps the inclusive
// cumulative sum G of log2|alpha| (fp32, each term clamped at -126) and the
// cumulative parity pi of negative gates; every ratio is
// (-1)^(pi_i ^ pi_j) 2^(G_i - G_j).
//
// A and P on matrix cores without overflow: tokens form four 16-token blocks.
// For a tile of row block I and column block J the row operand is scaled
// relative to the end of block I-1 (factor <= 1), the column operand relative
// to the end of block J (factor <= 1), and the per-channel bridge
// 2^(G_end(I-1) - G_end(J)) is <= 1 for J < I.  On the diagonal the bridge is
// >= 1; when any channel drops more than 2^100 inside a block, that block's
// tiles are computed element by element from the raw gates instead.
//
// Precision: every contraction whose operands are not raw bf16 inputs splits
// each fp32 operand x into hi = bf16(x) and lo = bf16(x - hi) and accumulates
// hi*hi + hi*lo + lo*hi in fp32 (three MFMAs), which keeps ~16 mantissa bits;
// T = (I + A)^-1 is formed in fp32 on the vector units (16 x 16 diagonal
// blocks by forward substitution, then three levels of block products).
//
// MFMA: v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, C 16x16).  Lane l holds
// A row l%16 / B column l%16 at k = 8(l/16) .. +7, and C rows 4(l/16) .. +3 of
// column l%16.  An accumulator used as the next product's B operand supplies
// rows {4g..4g+3, 16+4g..16+4g+3} of a 32-row k block (g = l/16); the matching
// A operand is read from LDS with the same k order.
#include "ckda_internal.h"

namespace ckda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;        // 64 tokens per chunk
constexpr int NT = 256;          // threads per workgroup (4 waves)
constexpr int BV = 64;           // dv columns per workgroup (16 per wave)
constexpr int RTS = C + 1;       // row stride of the fp32 A/T buffer
constexpr float kLog2Floor = -126.f;
constexpr float kDiagGuard = 100.f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// acc += a*b with a = ah + al, b = bh + bl, dropping al*bl.
__device__ __forceinline__ f32x4 mfma3(f32x4 c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
  c = mfma(al, bh, c);
  c = mfma(ah, bl, c);
  return mfma(ah, bh, c);
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &h, bf16x8 &l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 b = (__bf16)x[e];
    h[e] = b;
    l[e] = (__bf16)(x[e] - (float)b);
  }
}
__device__ __forceinline__ float sgn(uint32_t odd) { return odd ? -1.f : 1.f; }
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- LDS layout
// Rows are padded so that the fragment reads below are bank-conflict free
// while every address stays (per-lane base) + (compile-time offset): fp32
// [C][DK] regions by 16 bytes per row (16-byte reads of 8 consecutive rows hit
// distinct banks), bf16 planes by 8 bytes per row (8-byte reads of 16
// consecutive rows hit distinct banks).
constexpr int PADF = 4;          // fp32 row padding, elements
constexpr int PADB = 4;          // bf16 row padding, elements

template <int DK>
struct Lds {
  static constexpr int FR = C * (DK + PADF) * 4;          // fp32 [C][DK] region
  static constexpr int BQ = 2 * C * (DK + PADB) * 2;      // hi+lo planes [C][DK]
  static constexpr int BK = 2 * DK * (C + PADB) * 2;      // hi+lo planes [DK][C]
  static constexpr int BC = 2 * C * (C + PADB) * 2;       // hi+lo planes [C][C]
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  static constexpr int RA = 0;                            // Xk fp32 -> (-gamma K) planes
  static constexpr int RB = RA + mx(FR, BQ);              // Xq fp32 -> gamma Q planes
  static constexpr int RC = RB + mx(FR, BQ);              // Y fp32  -> K_hat^T planes
  static constexpr int RT = RC + mx(FR, BK);              // A, then T (fp32, stride C+1)
  static constexpr int RP = RT + C * RTS * 4;             // P fp32 [C][C] -> P planes
  static constexpr int RTB = RP + mx(C * C * 4, BC);      // T Diag(beta) planes; gate totals
  static constexpr int RZ = RTB + BC;                     // 3 x 16 x 16 fp32 scratch
  static constexpr int GE = RZ + 3 * 256 * 4;             // G at block ends [4][DK] fp32
  static constexpr int PE = GE + 4 * DK * 4;              // parity at block ends [4][DK] u8
  static constexpr int GN = PE + 4 * DK;                  // gamma_n [DK] fp32
  static constexpr int BT = GN + DK * 4;                  // beta [C] fp32
  static constexpr int FL = BT + C * 4;                   // diagonal-guard flags, 2 ints
  static constexpr int SIZE = FL + 16;
  static_assert(SIZE <= 160 * 1024, "LDS budget");
};

// element offsets
__device__ __forceinline__ int f32at(int row, int c, int DK) { return row * (DK + PADF) + c; }
__device__ __forceinline__ int bfat(int row, int c, int W) { return row * (W + PADB) + c; }

// A-operand fragment from a bf16 plane, k block kb, in the accumulator k order:
// channels 32kb + 4g .. +3 then 32kb + 16 + 4g .. +3.
__device__ __forceinline__ bf16x8 frag_acc_order(const __bf16 *plane, int W, int row, int kb,
                                                 int g) {
  const uint2 a = *reinterpret_cast<const uint2 *>(plane + bfat(row, 32 * kb + 4 * g, W));
  const uint2 b = *reinterpret_cast<const uint2 *>(plane + bfat(row, 32 * kb + 16 + 4 * g, W));
  uint4 u = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, u);
}
// B/C-fragment from two accumulator tiles (rows 0-15 and 16-31 of a k block).
__device__ __forceinline__ void frag_from_acc(const f32x4 &t0, const f32x4 &t1, bf16x8 &h,
                                              bf16x8 &l) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  split8(x, h, l);
}

template <int DK>
struct Geo {
  static constexpr int CQ = DK / 4;     // channel quads
  static constexpr int TG = NT / CQ;    // token groups
  static constexpr int TPT = C / TG;    // tokens per thread in the gate phase
  static_assert(TPT * TG == C && TPT % 4 == 0 && 16 % TPT == 0, "gate-phase geometry");
};

// Elementwise A and P for one diagonal block (the rare fallback).
template <int DK>
__device__ void diag_block_elementwise(int I, const __hip_bfloat16 *q, const __hip_bfloat16 *k,
                                       const float *g, const float *s_beta, size_t row0,
                                       size_t rstride, int nt, float *s_A, float *s_P) {
  for (int p = threadIdx.x; p < 256; p += NT) {
    const int a = p >> 4, b = p & 15;
    const int i = 16 * I + a, j = 16 * I + b;
    float accA = 0.f, accP = 0.f;
    if (b <= a && i < nt) {
      const size_t ri = row0 + (size_t)i * rstride, rj = row0 + (size_t)j * rstride;
      for (int c = 0; c < DK; ++c) {
        float r = 1.f;
        for (int s = j + 1; s <= i; ++s) {
          const float al = g[(row0 + (size_t)s * rstride) * DK + c];
          r *= copysignf(fmaxf(fabsf(al), 1.17549435e-38f), al);
        }
        const float kj = to_f32(k[rj * DK + c]) * r;
        accA += to_f32(k[ri * DK + c]) * kj;
        accP += to_f32(q[ri * DK + c]) * kj;
      }
    }
    s_A[i * RTS + j] = (b < a) ? s_beta[i] * accA : 0.f;
    s_P[i * C + j] = (b <= a) ? accP : 0.f;
  }
}

template <int DK>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_kernel(
    const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const float *__restrict__ S0, float *__restrict__ o,
    float *__restrict__ S_T, int T, int H, int DV, int NH, int NV, SeqTable tab, int packed) {
  using L = Lds<DK>;
  using GEO = Geo<DK>;
  constexpr int CQ = GEO::CQ, TPT = GEO::TPT, TG = GEO::TG;
  constexpr int KB = DK / 32;          // 32-channel k blocks
  constexpr int ST = DK / 16;          // 16-row state tiles per wave
  __shared__ __align__(16) char smem[L::SIZE];
  float *s_Xk = reinterpret_cast<float *>(smem + L::RA);
  float *s_Xq = reinterpret_cast<float *>(smem + L::RB);
  float *s_Y = reinterpret_cast<float *>(smem + L::RC);
  __bf16 *p_gk_h = reinterpret_cast<__bf16 *>(smem + L::RA);
  __bf16 *p_gk_l = p_gk_h + C * (DK + PADB);
  __bf16 *p_gq_h = reinterpret_cast<__bf16 *>(smem + L::RB);
  __bf16 *p_gq_l = p_gq_h + C * (DK + PADB);
  __bf16 *p_kh_h = reinterpret_cast<__bf16 *>(smem + L::RC);   // [DK][C]
  __bf16 *p_kh_l = p_kh_h + DK * (C + PADB);
  float *s_A = reinterpret_cast<float *>(smem + L::RT);
  float *s_P = reinterpret_cast<float *>(smem + L::RP);
  __bf16 *p_p_h = reinterpret_cast<__bf16 *>(smem + L::RP);
  __bf16 *p_p_l = p_p_h + C * (C + PADB);
  __bf16 *p_tb_h = reinterpret_cast<__bf16 *>(smem + L::RTB);
  __bf16 *p_tb_l = p_tb_h + C * (C + PADB);
  float *s_Gtot = reinterpret_cast<float *>(smem + L::RTB);              // [TG][DK]
  uint8_t *s_Ptot = reinterpret_cast<uint8_t *>(smem + L::RTB + TG * DK * 4);
  float *s_Z = reinterpret_cast<float *>(smem + L::RZ);
  float *s_GE = reinterpret_cast<float *>(smem + L::GE);
  uint8_t *s_PE = reinterpret_cast<uint8_t *>(smem + L::PE);
  float *s_GN = reinterpret_cast<float *>(smem + L::GN);
  float *s_beta = reinterpret_cast<float *>(smem + L::BT);
  int *s_flag = reinterpret_cast<int *>(smem + L::FL);

  // ---- which (sequence, head, dv block): XCD-aware.  Workgroup b runs on XCD
  // b % 8; the NV dv blocks of one (sequence, head) get the same XCD so they
  // share q/k/alpha in its L2, and low ranks (longest sequences) start first.
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int p = (slot / NV) * 8 + xcd, vb = slot % NV;
  if (p >= NH) return;
  const int rank = p / H, h = p % H;
  int n, start, len;
  if (packed) {
    n = tab.order[rank];
    start = tab.seq_start[n];
    len = tab.seq_len[n];
  } else {
    n = rank;
    start = n * T;
    len = T;
  }
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, gq = lane >> 4;
  const int col = vb * BV + 16 * w + l16;         // this lane's dv column
  const int cq = t % CQ, tg = t / CQ;              // gate phase: channel quad, token group
  const int c0 = 4 * cq, i0 = tg * TPT, blk = i0 >> 4;

  // ---- state slice in accumulators: tile tt holds rows 16tt + 4gq + e, column col.
  f32x4 accS[ST];
#pragma unroll
  for (int tt = 0; tt < ST; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      accS[tt][e] = S0 ? S0[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] : 0.f;

  if (t == 0) { s_flag[0] = 0; s_flag[1] = 0; }

  // ---- input loads for one chunk (issued a chunk ahead).
  float4 in_a[TPT];
  uint2 in_k[TPT], in_q[TPT];
  float in_b = 0.f;
  unsigned short in_v[4][4];
  auto load_chunk = [&](int lc) {
    const int t0 = start + lc * C, nt = min(C, len - lc * C);
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int i = i0 + r;
      if (i < nt) {
        const size_t row = (size_t)(t0 + i) * H + h;
        in_a[r] = *reinterpret_cast<const float4 *>(g + row * DK + c0);
        in_k[r] = *reinterpret_cast<const uint2 *>(k + row * DK + c0);
        in_q[r] = *reinterpret_cast<const uint2 *>(q + row * DK + c0);
      } else {
        in_a[r] = make_float4(1.f, 1.f, 1.f, 1.f);
        in_k[r] = make_uint2(0u, 0u);
        in_q[r] = make_uint2(0u, 0u);
      }
    }
    in_b = (t < C && t < nt) ? beta[(size_t)(t0 + t) * H + h] : 0.f;
    const unsigned short *vv = reinterpret_cast<const unsigned short *>(v);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + 4 * gq + e;
        in_v[mt][e] = i < nt ? vv[((size_t)(t0 + i) * H + h) * DV + col] : (unsigned short)0;
      }
  };

  const int nch = (len + C - 1) / C;
  if (nch > 0) load_chunk(0);
  __syncthreads();

  for (int lc = 0; lc < nch; ++lc) {
    const int t0 = start + lc * C, nt = min(C, len - lc * C);
    const size_t row0 = (size_t)t0 * H + h;
    // Re-derive the lane indices from an opaque copy of the thread id so that
    // the compiler recomputes per-chunk address arithmetic inside the loop
    // instead of keeping hundreds of hoisted addresses live across it.
    int t_opaque = threadIdx.x;
    asm volatile("" : "+v"(t_opaque));
    const int t = t_opaque, lane = t & 63, l16 = lane & 15, gq = lane >> 4;
    const int cq = t % CQ, tg = t / CQ, c0 = 4 * cq, i0 = tg * TPT, blk = i0 >> 4;
    const int col = vb * BV + 16 * w + l16;

    // ===================== P1: signed-gate scan (per channel, over tokens)
    // Gl: in-thread inclusive sums of log2|alpha|; pbits bit 4r+cc: in-thread
    // inclusive parity of negative gates for token r, channel cc.
    float Gl[TPT][4];
    uint32_t pbits = 0;
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const float a4[4] = {in_a[r].x, in_a[r].y, in_a[r].z, in_a[r].w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float lg = fmaxf(flog2(fabsf(a4[cc])), kLog2Floor);
        const uint32_t neg = a4[cc] < 0.f ? 1u : 0u;
        const uint32_t prev = r ? (pbits >> (4 * (r - 1) + cc)) & 1u : 0u;
        Gl[r][cc] = (r ? Gl[r - 1][cc] : 0.f) + lg;
        pbits |= (prev ^ neg) << (4 * r + cc);
      }
    }
    *reinterpret_cast<float4 *>(s_Gtot + tg * DK + c0) =
        make_float4(Gl[TPT - 1][0], Gl[TPT - 1][1], Gl[TPT - 1][2], Gl[TPT - 1][3]);
    *reinterpret_cast<uint32_t *>(s_Ptot + tg * DK + c0) =
        ((pbits >> (4 * (TPT - 1))) & 1u) | (((pbits >> (4 * (TPT - 1) + 1)) & 1u) << 8) |
        (((pbits >> (4 * (TPT - 1) + 2)) & 1u) << 16) | (((pbits >> (4 * (TPT - 1) + 3)) & 1u) << 24);
    if (t < C) s_beta[t] = in_b;
    __syncthreads();   // B1

    // prefix over token groups; block-end and chunk-end values per channel.
    // Gs/Ps: end of the block before this thread's block; Ge/Pe: end of it.
    float Gx[4], Gs[4], Ge[4], Gn[4];
    uint32_t Px[4], Ps[4], Pe[4], Pn[4];
    int myflag = 0;
    {
      float run[4] = {0.f, 0.f, 0.f, 0.f}, prev_end[4] = {0.f, 0.f, 0.f, 0.f};
      uint32_t prun = 0u;   // four parity bytes, one per channel of the quad
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        Gx[cc] = 0.f; Px[cc] = 0u; Gs[cc] = 0.f; Ps[cc] = 0u; Ge[cc] = 0.f; Pe[cc] = 0u;
      }
#pragma unroll
      for (int gg = 0; gg < TG; ++gg) {
        if (gg == tg) {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) { Gx[cc] = run[cc]; Px[cc] = (prun >> (8 * cc)) & 1u; }
        }
        const float4 gt = *reinterpret_cast<const float4 *>(s_Gtot + gg * DK + c0);
        run[0] += gt.x; run[1] += gt.y; run[2] += gt.z; run[3] += gt.w;
        prun ^= *reinterpret_cast<const uint32_t *>(s_Ptot + gg * DK + c0);
        if (((gg + 1) * TPT) % 16 == 0) {
          const int I = ((gg + 1) * TPT) / 16 - 1;     // block whose end this is
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            if (I == blk) { Ge[cc] = run[cc]; Pe[cc] = (prun >> (8 * cc)) & 1u; }
            if (I + 1 == blk) { Gs[cc] = run[cc]; Ps[cc] = (prun >> (8 * cc)) & 1u; }
            if (prev_end[cc] - run[cc] > kDiagGuard) myflag |= 1 << I;
            prev_end[cc] = run[cc];
          }
          if (tg == 0) {
            *reinterpret_cast<float4 *>(s_GE + I * DK + c0) = make_float4(run[0], run[1], run[2], run[3]);
            *reinterpret_cast<uint32_t *>(s_PE + I * DK + c0) = prun;
          }
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) { Gn[cc] = run[cc]; Pn[cc] = (prun >> (8 * cc)) & 1u; }
      if (tg == 0)
        *reinterpret_cast<float4 *>(s_GN + c0) =
            make_float4(sgn(Pn[0]) * fexp2(Gn[0]), sgn(Pn[1]) * fexp2(Gn[1]),
                        sgn(Pn[2]) * fexp2(Gn[2]), sgn(Pn[3]) * fexp2(Gn[3]));
      if (tg != 0) myflag = 0;
    }
    if (myflag) atomicOr(&s_flag[lc & 1], myflag);

    // row operands (relative to block start) and column operand (relative to block end)
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int i = i0 + r;
      const __hip_bfloat16 *kb16 = reinterpret_cast<const __hip_bfloat16 *>(&in_k[r]);
      const __hip_bfloat16 *qb16 = reinterpret_cast<const __hip_bfloat16 *>(&in_q[r]);
      float xk[4], xq[4], yk[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float G = Gx[cc] + Gl[r][cc];
        const uint32_t P = Px[cc] ^ ((pbits >> (4 * r + cc)) & 1u);
        const float ra = sgn(P ^ Ps[cc]) * fexp2(G - Gs[cc]);
        const float cb = sgn(Pe[cc] ^ P) * fexp2(Ge[cc] - G);
        const float kk = __bfloat162float(kb16[cc]);
        xk[cc] = kk * ra;
        xq[cc] = __bfloat162float(qb16[cc]) * ra;
        yk[cc] = kk * cb;
      }
      *reinterpret_cast<float4 *>(s_Xk + f32at(i, c0, DK)) = make_float4(xk[0], xk[1], xk[2], xk[3]);
      *reinterpret_cast<float4 *>(s_Xq + f32at(i, c0, DK)) = make_float4(xq[0], xq[1], xq[2], xq[3]);
      *reinterpret_cast<float4 *>(s_Y + f32at(i, c0, DK)) = make_float4(yk[0], yk[1], yk[2], yk[3]);
    }
    if (t == 0) s_flag[(lc + 1) & 1] = 0;
    __syncthreads();   // B2
    const int flags = s_flag[lc & 1];

    // ===================== P3: A and P tiles on matrix cores
    {
      // ten (I, J) tile pairs, J <= I: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
      for (int pr = w; pr < 10; pr += 4) {
        const int I = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
        const int J = pr - I * (I + 1) / 2;
        const bool diag = I == J;
        if (diag && ((flags >> I) & 1)) continue;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) {
          const int c = 32 * ks + 8 * gq;
          const int ri = 16 * I + l16, rj = 16 * J + l16;
          float xk[8], xq[8], y[8];
          *reinterpret_cast<float4 *>(xk) = *reinterpret_cast<const float4 *>(s_Xk + f32at(ri, c, DK));
          *reinterpret_cast<float4 *>(xk + 4) = *reinterpret_cast<const float4 *>(s_Xk + f32at(ri, c + 4, DK));
          *reinterpret_cast<float4 *>(xq) = *reinterpret_cast<const float4 *>(s_Xq + f32at(ri, c, DK));
          *reinterpret_cast<float4 *>(xq + 4) = *reinterpret_cast<const float4 *>(s_Xq + f32at(ri, c + 4, DK));
          *reinterpret_cast<float4 *>(y) = *reinterpret_cast<const float4 *>(s_Y + f32at(rj, c, DK));
          *reinterpret_cast<float4 *>(y + 4) = *reinterpret_cast<const float4 *>(s_Y + f32at(rj, c + 4, DK));
          float gs[8], ge[8];
          uint2 ps = {0u, 0u};
          if (I) {
            *reinterpret_cast<float4 *>(gs) = *reinterpret_cast<const float4 *>(s_GE + (I - 1) * DK + c);
            *reinterpret_cast<float4 *>(gs + 4) = *reinterpret_cast<const float4 *>(s_GE + (I - 1) * DK + c + 4);
            ps = *reinterpret_cast<const uint2 *>(s_PE + (I - 1) * DK + c);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gs[e] = 0.f;
          }
          *reinterpret_cast<float4 *>(ge) = *reinterpret_cast<const float4 *>(s_GE + J * DK + c);
          *reinterpret_cast<float4 *>(ge + 4) = *reinterpret_cast<const float4 *>(s_GE + J * DK + c + 4);
          const uint2 pe = *reinterpret_cast<const uint2 *>(s_PE + J * DK + c);
          const uint32_t par_lo = ps.x ^ pe.x, par_hi = ps.y ^ pe.y;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t odd = ((e < 4 ? par_lo : par_hi) >> (8 * (e & 3))) & 1u;
            const float D = sgn(odd) * fexp2(gs[e] - ge[e]);
            xk[e] *= D;
            xq[e] *= D;
          }
          bf16x8 akh, akl, aqh, aql, yh, yl;
          split8(xk, akh, akl);
          split8(xq, aqh, aql);
          split8(y, yh, yl);
          accA = mfma3(accA, akh, akl, yh, yl);
          accP = mfma3(accP, aqh, aql, yh, yl);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * I + 4 * gq + e, j = 16 * J + l16;
          s_A[i * RTS + j] = (!diag || j < i) ? s_beta[i] * accA[e] : 0.f;
          s_P[i * C + j] = (!diag || j <= i) ? accP[e] : 0.f;
        }
      }
      // zero P above the diagonal blocks
      for (int x = t; x < 6 * 256; x += NT) {
        // blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int bi = x >> 8, e = x & 255;
        const int ui = bi < 3 ? 0 : bi < 5 ? 1 : 2;
        const int uj = bi < 3 ? bi + 1 : bi < 5 ? bi - 1 : 3;
        s_P[(16 * ui + (e >> 4)) * C + 16 * uj + (e & 15)] = 0.f;
      }
    }
    __syncthreads();   // B3
    if (flags) {
#pragma unroll 1
      for (int I = 0; I < 4; ++I)
        if ((flags >> I) & 1)
          diag_block_elementwise<DK>(I, q, k, g, s_beta, row0, (size_t)H, nt, s_A, s_P);
      __syncthreads();
    }

    // ===================== P4: matrix-core operands for the state pass,
    // T diagonal blocks (wave 0), P to registers
    // Own Xk, Xq, Y back from LDS; they are rewritten as bf16 planes after B4.
    float4 rXk[TPT], rXq[TPT], rY[TPT];
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      rXk[r] = *reinterpret_cast<const float4 *>(s_Xk + f32at(i0 + r, c0, DK));
      rXq[r] = *reinterpret_cast<const float4 *>(s_Xq + f32at(i0 + r, c0, DK));
      rY[r] = *reinterpret_cast<const float4 *>(s_Y + f32at(i0 + r, c0, DK));
    }
    if (w == 0) {
      // (I + A_II)^-1 for the four diagonal blocks; lane = 16 I + column
      const int I = lane >> 4, j = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s -= s_A[(16 * I + i) * RTS + 16 * I + m] * x[m];
        x[i] = (i < j) ? 0.f : s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s_A[(16 * I + i) * RTS + 16 * I + j] = x[i];
    }
    float pv[16];
    {
      const int pi = t >> 2, pj = (t & 3) * 16;
#pragma unroll
      for (int u = 0; u < 16; u += 4)
        *reinterpret_cast<float4 *>(pv + u) = *reinterpret_cast<const float4 *>(s_P + pi * C + pj + u);
    }
    __syncthreads();   // B4
    {
      float gam_s[4], del_e[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        gam_s[cc] = sgn(Ps[cc]) * fexp2(Gs[cc]);                          // chunk start -> block start
        del_e[cc] = sgn(Pe[cc] ^ Pn[cc]) * fexp2(Gn[cc] - Ge[cc]);        // block end -> chunk end
      }
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const int i = i0 + r;
        const float xk[4] = {rXk[r].x, rXk[r].y, rXk[r].z, rXk[r].w};
        const float xq[4] = {rXq[r].x, rXq[r].y, rXq[r].z, rXq[r].w};
        __bf16 hk[4], lk[4], hq[4], lq[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float a = -xk[cc] * gam_s[cc];     // -(gamma K)
          const float bq = xq[cc] * gam_s[cc];     // gamma Q
          hk[cc] = (__bf16)a; lk[cc] = (__bf16)(a - (float)hk[cc]);
          hq[cc] = (__bf16)bq; lq[cc] = (__bf16)(bq - (float)hq[cc]);
        }
        *reinterpret_cast<uint2 *>(p_gk_h + bfat(i, c0, DK)) = __builtin_bit_cast(uint2, hk);
        *reinterpret_cast<uint2 *>(p_gk_l + bfat(i, c0, DK)) = __builtin_bit_cast(uint2, lk);
        *reinterpret_cast<uint2 *>(p_gq_h + bfat(i, c0, DK)) = __builtin_bit_cast(uint2, hq);
        *reinterpret_cast<uint2 *>(p_gq_l + bfat(i, c0, DK)) = __builtin_bit_cast(uint2, lq);
      }
      // K_hat^T = (K gamma_n / gamma)^T, [channel][token]
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int r4 = 0; r4 < TPT; r4 += 4) {
          __bf16 hh[4], ll[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float y4[4] = {rY[r4 + u].x, rY[r4 + u].y, rY[r4 + u].z, rY[r4 + u].w};
            const float x = y4[cc] * del_e[cc];
            hh[u] = (__bf16)x; ll[u] = (__bf16)(x - (float)hh[u]);
          }
          *reinterpret_cast<uint2 *>(p_kh_h + bfat(c0 + cc, i0 + r4, C)) = __builtin_bit_cast(uint2, hh);
          *reinterpret_cast<uint2 *>(p_kh_l + bfat(c0 + cc, i0 + r4, C)) = __builtin_bit_cast(uint2, ll);
        }
      }
    }
    {
      const int pi = t >> 2, pj = (t & 3) * 16;
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        __bf16 hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hh[e] = (__bf16)pv[u + e];
          ll[e] = (__bf16)(pv[u + e] - (float)hh[e]);
        }
        *reinterpret_cast<uint2 *>(p_p_h + bfat(pi, pj + u, C)) = __builtin_bit_cast(uint2, hh);
        *reinterpret_cast<uint2 *>(p_p_l + bfat(pi, pj + u, C)) = __builtin_bit_cast(uint2, ll);
      }
    }

    // ===================== P5: off-diagonal blocks of T, three levels.
    // T_IJ (I > J) is stored in the free upper block (J, I) of the A/T buffer.
    auto Tdiag = [&](int I, int a, int bb) { return s_A[(16 * I + a) * RTS + 16 * I + bb]; };
    auto Toff = [&](int I, int J, int a, int bb) { return s_A[(16 * J + a) * RTS + 16 * I + bb]; };
    auto Aof = [&](int I, int J, int a, int bb) { return s_A[(16 * I + a) * RTS + 16 * J + bb]; };
#pragma unroll 1
    for (int lev = 1; lev <= 3; ++lev) {
      const int ntile = 4 - lev;
      for (int x = t; x < ntile * 256; x += NT) {
        const int J = x >> 8, a = (x >> 4) & 15, bb = x & 15, I = J + lev;
        float z = 0.f;
        for (int M = J; M < I; ++M)
#pragma unroll
          for (int m = 0; m < 16; ++m)
            z += Aof(I, M, a, m) * (M == J ? Tdiag(J, m, bb) : Toff(M, J, m, bb));
        s_Z[x] = z;
      }
      __syncthreads();
      for (int x = t; x < ntile * 256; x += NT) {
        const int J = x >> 8, a = (x >> 4) & 15, bb = x & 15, I = J + lev;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s += Tdiag(I, a, m) * s_Z[(J << 8) + (m << 4) + bb];
        s_A[(16 * J + a) * RTS + 16 * I + bb] = -s;
      }
      __syncthreads();
    }
    // T Diag(beta) -> hi/lo planes (zero above the diagonal)
    {
      const int i = t >> 2, j0 = (t & 3) * 16, I = i >> 4, a = i & 15;
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        __bf16 hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + u + e, J = j >> 4, bb = j & 15;
          float tv = 0.f;
          if (J == I) tv = bb <= a ? Tdiag(I, a, bb) : 0.f;
          else if (J < I) tv = Toff(I, J, a, bb);
          tv *= s_beta[j];
          hh[e] = (__bf16)tv;
          ll[e] = (__bf16)(tv - (float)hh[e]);
        }
        *reinterpret_cast<uint2 *>(p_tb_h + bfat(i, j0 + u, C)) = __builtin_bit_cast(uint2, hh);
        *reinterpret_cast<uint2 *>(p_tb_l + bfat(i, j0 + u, C)) = __builtin_bit_cast(uint2, ll);
      }
    }
    __syncthreads();   // B5

    // ===================== state pass (each wave: 16 columns, all tokens)
    unsigned short cur_v[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) cur_v[mt][e] = in_v[mt][e];
    if (lc + 1 < nch) load_chunk(lc + 1);     // prefetch the next chunk

    bf16x8 sh[KB], sl[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) frag_from_acc(accS[2 * kb], accS[2 * kb + 1], sh[kb], sl[kb]);

    // X = V - (gamma K) S
    f32x4 accX[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accX[mt][e] = __bfloat162float(__builtin_bit_cast(__hip_bfloat16, cur_v[mt][e]));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ah = frag_acc_order(p_gk_h, DK, 16 * mt + l16, kb, gq);
        const bf16x8 al = frag_acc_order(p_gk_l, DK, 16 * mt + l16, kb, gq);
        accX[mt] = mfma3(accX[mt], ah, al, sh[kb], sl[kb]);
      }
    }
    bf16x8 xh[2], xl[2];
    frag_from_acc(accX[0], accX[1], xh[0], xl[0]);
    frag_from_acc(accX[2], accX[3], xh[1], xl[1]);

    // U = T Diag(beta) X   (lower triangular: row tile mt needs k blocks <= mt/2)
    f32x4 accU[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      accU[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= (mt >> 1); ++kb) {
        const bf16x8 ah = frag_acc_order(p_tb_h, C, 16 * mt + l16, kb, gq);
        const bf16x8 al = frag_acc_order(p_tb_l, C, 16 * mt + l16, kb, gq);
        accU[mt] = mfma3(accU[mt], ah, al, xh[kb], xl[kb]);
      }
    }
    bf16x8 uh[2], ul[2];
    frag_from_acc(accU[0], accU[1], uh[0], ul[0]);
    frag_from_acc(accU[2], accU[3], uh[1], ul[1]);

    // O = (gamma Q) S + P U
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ah = frag_acc_order(p_gq_h, DK, 16 * mt + l16, kb, gq);
        const bf16x8 al = frag_acc_order(p_gq_l, DK, 16 * mt + l16, kb, gq);
        acc = mfma3(acc, ah, al, sh[kb], sl[kb]);
      }
#pragma unroll
      for (int kb = 0; kb <= (mt >> 1); ++kb) {
        const bf16x8 ah = frag_acc_order(p_p_h, C, 16 * mt + l16, kb, gq);
        const bf16x8 al = frag_acc_order(p_p_l, C, 16 * mt + l16, kb, gq);
        acc = mfma3(acc, ah, al, uh[kb], ul[kb]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + 4 * gq + e;
        if (i < nt) o[((size_t)(t0 + i) * H + h) * DV + col] = acc[e];
      }
    }

    // S <- Diag(gamma_n) S + K_hat^T U
#pragma unroll
    for (int tt = 0; tt < ST; ++tt) {
      const float4 gn = *reinterpret_cast<const float4 *>(s_GN + 16 * tt + 4 * gq);
      accS[tt][0] *= gn.x; accS[tt][1] *= gn.y; accS[tt][2] *= gn.z; accS[tt][3] *= gn.w;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ah = frag_acc_order(p_kh_h, C, 16 * tt + l16, kb, gq);
        const bf16x8 al = frag_acc_order(p_kh_l, C, 16 * tt + l16, kb, gq);
        accS[tt] = mfma3(accS[tt], ah, al, uh[kb], ul[kb]);
      }
    }
    __syncthreads();   // B6: LDS operands are rewritten by the next chunk
  }

  if (S_T) {
#pragma unroll
    for (int tt = 0; tt < ST; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_T[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] = accS[tt][e];
  }
}

template <int DK>
hipError_t launch_dk(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *S0, float *o, float *S_T, int T, int H,
                     int DV, int N, SeqTable tab, int packed, hipStream_t stream) {
  const int NH = N * H, NV = DV / BV;
  const int groups = (NH + 7) / 8;
  const dim3 grid((unsigned)groups * 8u * (unsigned)NV), block(NT);
  hipLaunchKernelGGL((fwd_bf16_kernel<DK>), grid, block, 0, stream,
                     static_cast<const __hip_bfloat16 *>(q), static_cast<const __hip_bfloat16 *>(k),
                     static_cast<const __hip_bfloat16 *>(v), g, beta, S0, o, S_T, T, H, DV, NH, NV,
                     tab, packed);
  return hipGetLastError();
}

}  // namespace

size_t fwd_bf16_lds_bytes(int dk) { return dk == 64 ? Lds<64>::SIZE : Lds<128>::SIZE; }

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, float *o, float *S_T, int T, int H,
                           int dk, int dv, int N, SeqTable tab, int packed, hipStream_t stream) {
  if (dk == 64)
    return launch_dk<64>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, packed, stream);
  if (dk == 128)
    return launch_dk<128>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, packed, stream);
  return hipErrorInvalidValue;
}

}  // namespace ckda
