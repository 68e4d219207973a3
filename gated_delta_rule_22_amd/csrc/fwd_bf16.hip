// Fused chunkwise CKDA forward for bf16 q/k/v on CDNA4 matrix cores.
//
// One workgroup owns one (sequence, head, 64-column block of dv) and walks the
// sequence's chunks of C = 64 tokens in order.  Its slice of the fp32 state
// (dk x 64) lives in MFMA accumulators for the whole sequence; each chunk is
// read from HBM once (the dv blocks of a head share q/k/alpha through the L2
// of their XCD) and o is written once, so the HBM traffic is the compulsory one.
//
// Chunk algebra (update rule: blog post "One update, one quarter turn", ELI5
// "The mirror", unrolled over a chunk with incoming state S; gamma_i is the
// product of the gates of tokens 1..i of the chunk, per key channel):
//   A_ij = beta_i sum_c (gamma_ic k_ic) (k_jc / gamma_jc)      (i > j)
//   P_ij =        sum_c (gamma_ic q_ic) (k_jc / gamma_jc)      (j <= i)
//   X    = V - (gamma K) S,   (I + A) U = Diag(beta) X
//   O    = (gamma Q) S + P U
//   S'   = Diag(gamma_n) S + (K gamma_n / gamma)^T U
//
// Signed gates (CKDA summary, "Methodology in Plain English": gate magnitudes
// live in log space, so the sign is kept apart): per channel the chunk keeps
// the inclusive cumulative sum G of log2|alpha| (fp32, each term clamped at
// -126) and the cumulative parity pi of negative gates.  Only ratios of gammas
// matter, so each channel is referenced to R = G_n / 2, the middle of its
// range: gamma' = (-1)^pi 2^(G - R) and 1/gamma' = (-1)^pi 2^(R - G) both stay
// within 2^+-100 while the chunk's log-gate range is below 200 (gates averaging
// above 0.11 in magnitude), and A, P are one product each of gamma'-scaled
// operands.  The state absorbs 2^R: with S_pre = 2^R S,
//   X = V - (gamma' K) S_pre,  O = (gamma' Q) S_pre + P U,
//   S' = (-1)^pi_n 2^(G_n - R) (S_pre + (K / gamma')^T U).
// A chunk whose range is wider takes an exact element-wise path that only
// forms 2^(G_i - G_j) <= 1.
//
// Work split inside the workgroup (512 threads):
//   waves 0-3  state pass, 16 dv columns each: X, O, U and the state update,
//              all on matrix cores; wave 0 also inverts the diagonal blocks;
//   waves 4-7  chunk preparation for the next chunk while the state pass runs:
//              gate scan, gamma'-scaled operands and their hi/lo bf16 split;
//              at the hand-off, A and P on matrix cores.
// (I + A) U = Diag(beta) X is solved by block forward substitution over the
// four 16-token blocks, so T = (I + A)^-1 is never formed.
//
// Precision: every contraction whose operands are not raw bf16 inputs splits
// each fp32 operand x into hi = bf16(x) and lo = bf16(x - hi) and accumulates
// hi*hi + hi*lo + lo*hi in fp32 (three MFMAs), keeping ~16 mantissa bits.
//
// MFMA shapes (lane l, g = l / 16):
//   16x16x32: A row l%16 / B column l%16 hold k = 8g .. 8g+7; C rows 4g..4g+3.
//     An accumulator pair used as a B operand supplies k rows
//     {4g..4g+3, 16+4g..16+4g+3}; the matching A operand is read in that order.
//   16x16x16: A row / B column l%16 hold k = 4g .. 4g+3, the accumulator layout,
//     so a 16-token accumulator is directly the next product's B operand.
#include "ckda_internal.h"

namespace ckda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int C = kChunk;        // 64 tokens per chunk
constexpr int NT = 512;          // 8 waves per workgroup
constexpr int BV = 64;           // dv columns per workgroup (16 per state-pass wave)
constexpr int PADB = 4;          // bf16 plane row padding (elements)
constexpr int ADS = 20;          // row stride of the fp32 diagonal A tiles (16-byte rows)
constexpr int ADB = 16 * ADS + 4; // block stride: the four blocks start on different banks
constexpr float kLog2Floor = -126.f;
constexpr float kGuard = 100.f;  // |G - R| bound for the factored A and P
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: raw 32-bit data

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// acc += a*b with a = ah + al, b = bh + bl (al*bl dropped).
__device__ __forceinline__ f32x4 mfma32x3(f32x4 c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
  c = mfma32(al, bh, c);
  c = mfma32(ah, bl, c);
  return mfma32(ah, bh, c);
}
__device__ __forceinline__ f32x4 mfma16x3(f32x4 c, bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl) {
  c = mfma16(al, bh, c);
  c = mfma16(ah, bl, c);
  return mfma16(ah, bh, c);
}
// Padding between a 16x16x16 bf16 product and the vector instructions that
// read its accumulator.  On gfx950 the wait states the compiler inserts there
// were measured too few: the first registers of the result were read stale.
// Sixteen idle cycles, fenced so that no instruction moves across them.
__device__ __forceinline__ void settle16() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void split1(float x, __bf16 &h, __bf16 &l) {
  h = (__bf16)x;
  l = (__bf16)(x - (float)h);
}
// hi/lo split of two fp32 values into packed bf16 pairs (round to nearest
// even on both parts), with one packed conversion for each part.
__device__ __forceinline__ void split2(float a, float b, uint32_t &h, uint32_t &l) {
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  const float ra = a - __builtin_bit_cast(float, hb << 16);
  const float rb = b - __builtin_bit_cast(float, hb & 0xFFFF0000u);
  h = hb;
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
}
__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &h, bf16x4 &l) {
  uint2 hh, ll;
  split2(x[0], x[1], hh.x, ll.x);
  split2(x[2], x[3], hh.y, ll.y);
  h = __builtin_bit_cast(bf16x4, hh);
  l = __builtin_bit_cast(bf16x4, ll);
}
// k-block fragment of two accumulator tiles (rows 0-15 and 16-31 of a 32-row block)
__device__ __forceinline__ void split8_acc(const f32x4 &t0, const f32x4 &t1, bf16x8 &h,
                                           bf16x8 &l) {
  uint4 hh, ll;
  split2(t0[0], t0[1], hh.x, ll.x);
  split2(t0[2], t0[3], hh.y, ll.y);
  split2(t1[0], t1[1], hh.z, ll.z);
  split2(t1[2], t1[3], hh.w, ll.w);
  h = __builtin_bit_cast(bf16x8, hh);
  l = __builtin_bit_cast(bf16x8, ll);
}
// hi/lo split of four fp32 values into packed bf16 pairs (round to nearest
// even on both parts): x = hi + lo + O(2^-17 |x|).
__device__ __forceinline__ void split_quad(const float (&x)[4], uint2 &h, uint2 &l) {
  uint32_t hw[2], lw[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const bf16x2 hp = __builtin_convertvector((f32x2){x[2 * p], x[2 * p + 1]}, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, hp);
    const float r0 = x[2 * p] - __builtin_bit_cast(float, hb << 16);
    const float r1 = x[2 * p + 1] - __builtin_bit_cast(float, hb & 0xFFFF0000u);
    hw[p] = hb;
    lw[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
  }
  h = make_uint2(hw[0], hw[1]);
  l = make_uint2(lw[0], lw[1]);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float with_sign(float x, uint32_t odd) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) ^ (odd << 31));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// ---------------------------------------------------------------- LDS layout
// bf16 hi/lo planes; rows padded by 8 bytes so the 8-byte fragment reads of 16
// consecutive rows hit distinct banks while every address stays (per-lane base)
// + (compile-time offset).
template <int DK>
struct Lds {
  static constexpr int PQ = 2 * C * (DK + PADB) * 2;      // hi+lo [C][DK]
  static constexpr int PT = 2 * DK * (C + PADB) * 2;      // hi+lo [DK][C]
  static constexpr int PC = 2 * C * (C + PADB) * 2;       // hi+lo [C][C]
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  static constexpr int GK = 0;                            // -(gamma K)       [C][DK]
  static constexpr int GQ = GK + PQ;                      // gamma Q          [C][DK]
  static constexpr int KT = GQ + PQ;                      // (K/gamma)^T      [DK][C]
  static constexpr int P = KT + PT;                       // P                [C][C]
  static constexpr int KG = P + PC;                       // K/gamma [C][DK]; then AT
  static constexpr int AT = KG;                           // -A below, T_II on the diagonal
  static constexpr int FG = C * DK * 4;                   // exact path: G fp32 [C][DK]
  static constexpr int KG_BYTES = mx(mx(PQ, PC), FG + DK * 8);
  static constexpr int AD = KG + KG_BYTES;                // diagonal A tiles fp32 [4][16][20]
  static constexpr int BT = AD + 4 * ADB * 4;             // beta [C]
  static constexpr int SPRE = BT + C * 4;                 // S_pre = pre * S          [DK]
  static constexpr int SMID = SPRE + DK * 4;              // S' = post * (mid * S_pre  [DK]
  static constexpr int SPOST = SMID + DK * 4;             //      + (KT plane)^T U)    [DK]
  static constexpr int FL = SPOST + DK * 4;               // guard flags (2 ints)
  static constexpr int NRM = FL + 16;                     // q/k norm partials [4][C][2]
  static constexpr int FAC = NRM + 4 * C * 8;             // q/k norm factors  [C][2]
  static constexpr int SIZE = FAC + C * 8;
  static_assert(SIZE <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int at(int row, int c, int W) { return row * (W + PADB) + c; }

// 16x16x32 A-operand fragment in the accumulator k order (see header).
__device__ __forceinline__ bf16x8 frag32(const __bf16 *plane, int W, int row, int kb, int g) {
  const uint2 a = *reinterpret_cast<const uint2 *>(plane + at(row, 32 * kb + 4 * g, W));
  const uint2 b = *reinterpret_cast<const uint2 *>(plane + at(row, 32 * kb + 16 + 4 * g, W));
  const uint4 u = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, u);
}
// 16x16x16 A-operand fragment: columns col0 + 4g .. +3 of `row`.
__device__ __forceinline__ bf16x4 frag16(const __bf16 *plane, int W, int row, int col0, int g) {
  return __builtin_bit_cast(bf16x4,
                            *reinterpret_cast<const uint2 *>(plane + at(row, col0 + 4 * g, W)));
}

// A per-lane LDS byte offset the compiler must keep in a register: reads at
// (offset + compile-time constant) then fold the constant into the
// instruction's 16-bit offset field instead of recomputing the address.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
template <class T>
__device__ __forceinline__ T lds_at(const char *smem, int base, int imm) {
  return *reinterpret_cast<const T *>(smem + base + imm);
}
// 16x16x32 fragment (accumulator k order) at byte base + imm: the lane's
// columns 4g..4g+3 and 16+4g..16+4g+3 of a 32-column block.
__device__ __forceinline__ bf16x8 frag32o(const char *smem, int base, int imm) {
  const uint2 a = lds_at<uint2>(smem, base, imm);
  const uint2 b = lds_at<uint2>(smem, base, imm + 32);
  const uint4 u = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ bf16x4 frag16o(const char *smem, int base, int imm) {
  return __builtin_bit_cast(bf16x4, lds_at<uint2>(smem, base, imm));
}
// byte offset of (row, col) in a bf16 plane of width W (padded rows)
constexpr int pb(int row, int col, int W) { return 2 * (row * (W + PADB) + col); }

template <int DK>
struct Prep {                     // chunk-preparation lane geometry (one wave: DK/4 channels)
  static constexpr int CQW = DK / 16;     // channel quads per wave
  static constexpr int TGW = 64 / CQW;    // token groups per wave
  static constexpr int TPL = C / TGW;     // tokens per lane
  static_assert(TPL * TGW == C && TPL % 4 == 0, "preparation geometry");
};

__device__ __forceinline__ void tile_of_pair(int pr, int &I, int &J) {
  // ten (I, J) tile pairs with J <= I: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
  I = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
  J = pr - I * (I + 1) / 2;
}

// ---------------------------------------------------------------- kernel
// SIGNED: CKDA (false: KDA mode, gate signs ignored).  NORM: q and k are
// L2-normalised per (token, head) on the fly.  OBF16: o is written as bf16.
template <int DK, bool SIGNED, bool NORM, bool OBF16>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_kernel(
    const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const float *S0, void *__restrict__ o,
    float *S_T, int T, int H, int DV, int NH, int NV, SeqTable tab, int packed) {
  using L = Lds<DK>;
  using PG = Prep<DK>;
  constexpr int CQW = PG::CQW, TGW = PG::TGW, TPL = PG::TPL;
  constexpr int KB = DK / 32;     // 32-channel k blocks
  constexpr int ST = DK / 16;     // 16-row state tiles per state-pass wave
  __shared__ __align__(16) char smem[L::SIZE];
  __bf16 *gk_h = reinterpret_cast<__bf16 *>(smem + L::GK), *gk_l = gk_h + C * (DK + PADB);
  __bf16 *gq_h = reinterpret_cast<__bf16 *>(smem + L::GQ), *gq_l = gq_h + C * (DK + PADB);
  __bf16 *kt_h = reinterpret_cast<__bf16 *>(smem + L::KT), *kt_l = kt_h + DK * (C + PADB);
  __bf16 *kg_h = reinterpret_cast<__bf16 *>(smem + L::KG), *kg_l = kg_h + C * (DK + PADB);
  __bf16 *p_h = reinterpret_cast<__bf16 *>(smem + L::P), *p_l = p_h + C * (C + PADB);
  __bf16 *at_h = reinterpret_cast<__bf16 *>(smem + L::AT), *at_l = at_h + C * (C + PADB);
  float *s_ad = reinterpret_cast<float *>(smem + L::AD);
  float *s_beta = reinterpret_cast<float *>(smem + L::BT);
  float *s_pre = reinterpret_cast<float *>(smem + L::SPRE);
  float *s_mid = reinterpret_cast<float *>(smem + L::SMID);
  float *s_post = reinterpret_cast<float *>(smem + L::SPOST);
  int *s_flag = reinterpret_cast<int *>(smem + L::FL);
  float *s_nrm = reinterpret_cast<float *>(smem + L::NRM);
  float *s_fac = reinterpret_cast<float *>(smem + L::FAC);

  // ---- which (sequence, head, dv block): XCD-aware.  Workgroup b runs on XCD
  // b % 8; the NV dv blocks of one (sequence, head) share an XCD (and its L2),
  // and low ranks (the longest sequences when packed) start first.
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int pidx = (slot / NV) * 8 + xcd, vb = slot % NV;
  if (pidx >= NH) return;
  const int rank = pidx / H, h = pidx % H;
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
  const int nch = (len + C - 1) / C;
  const int w = threadIdx.x >> 6;
  const bool prep = w >= 4;           // chunk-preparation wave

  // ---- state-pass lane state
  f32x4 accS[ST];
  unsigned short in_v[4][4];
  // ---- preparation lane state
  float4 in_a[TPL];
  uint2 in_k[TPL], in_q[TPL];
  float in_b = 0.f;
  uint2 o_kg_h[TPL], o_kg_l[TPL];
  float pre4[4], post4[4];
  uint32_t guard_bad = 0;

  // Global traffic goes through buffer resources based at a chunk's first
  // token row, with num_records ending at the sequence's last row of this head:
  // rows past the sequence end read as zero and writes to them are dropped, so
  // no lane branches or clamps, and per-token offsets stay 32-bit.
  auto rsrc = [&](const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, kBufferFlags);
  };
  auto sp_load_v = [&](int lc, int tpin) {
    const int lane = tpin & 63, gq = lane >> 4;
    const int col = vb * BV + 16 * (tpin >> 6) + (lane & 15);
    const int t0 = start + lc * C, nt = min(C, len - lc * C);
    const int rs = H * DV * 2;
    const auto rv = rsrc(v + ((size_t)t0 * H + h) * DV, (nt - 1) * rs + DV * 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        in_v[mt][e] = __builtin_amdgcn_raw_buffer_load_b16(rv, (16 * mt + 4 * gq + e) * rs + 2 * col, 0, 0);
  };
  // part 0: the gates; part 1: keys, queries and beta; 2: both.  The next
  // chunk's two halves are issued in different phases, so the issue cost of
  // 16 KB of loads per wave is not paid in one stretch.
  auto pr_load = [&](int lc, int tpin, int part) {
    const int lane = tpin & 63, pw = (tpin >> 6) - 4;
    const int c0 = 4 * (pw * CQW + lane % CQW), i0 = (lane / CQW) * TPL;
    const int t0 = start + lc * C, nt = min(C, len - lc * C);
    const size_t row0 = (size_t)t0 * H + h;
    const int rsg = H * DK * 4, rsk = H * DK * 2;
    if (part != 1) {
      const auto rg = rsrc(g + row0 * DK, (nt - 1) * rsg + DK * 4);
#pragma unroll
      for (int r = 0; r < TPL; ++r)
        in_a[r] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, (i0 + r) * rsg + 4 * c0, 0, 0));
    }
    if (part != 0) {
      const auto rk = rsrc(k + row0 * DK, (nt - 1) * rsk + DK * 2);
      const auto rq = rsrc(q + row0 * DK, (nt - 1) * rsk + DK * 2);
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        in_k[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, (i0 + r) * rsk + 2 * c0, 0, 0));
        in_q[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, (i0 + r) * rsk + 2 * c0, 0, 0));
      }
      const auto rb = rsrc(beta + row0, (nt - 1) * H * 4 + 4);
      in_b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
    }
  };

  // Squared norms of the prefetched keys and queries over this wave's channels,
  // summed over the lanes of each token group; the four waves' partials meet in
  // LDS at the next barrier.
  auto pr_partials = [&](int tpin) {
    const int lane = tpin & 63, pw = (tpin >> 6) - 4;
    const int cql = lane % CQW, i0 = (lane / CQW) * TPL;
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint32_t kw = cc < 2 ? in_k[r].x : in_k[r].y, qw = cc < 2 ? in_q[r].x : in_q[r].y;
        const float kk = __builtin_bit_cast(float, (cc & 1) ? (kw & 0xFFFF0000u) : (kw << 16));
        const float qq = __builtin_bit_cast(float, (cc & 1) ? (qw & 0xFFFF0000u) : (qw << 16));
        pk += kk * kk;
        pq += qq * qq;
      }
#pragma unroll
      for (int m = 1; m < CQW; m <<= 1) {
        pk += __shfl_xor(pk, m);
        pq += __shfl_xor(pq, m);
      }
      if (cql == 0)
        *reinterpret_cast<float2 *>(s_nrm + (pw * C + i0 + r) * 2) = make_float2(pk, pq);
    }
  };

  // Register stage of chunk preparation: gate scan across the wave's lanes,
  // gamma'-scaled operands and their hi/lo split.  -(gamma' K) and gamma' Q go
  // straight to LDS (the state pass is done with those planes once H4 has
  // passed); K/gamma' is held for the hand-off.
  //
  // The running log-gate is kept as m = -G >= 0 with the gate-sign parity in
  // the sign bit of the same fp32 word, so one word per (token, channel) holds
  // both and |m| reads the magnitude for free.
  auto pr_compute = [&](int nt_c) {
    int t_opaque = threadIdx.x;
    asm volatile("" : "+v"(t_opaque));
    const int lane = t_opaque & 63, tg = lane / CQW, cql = lane % CQW;
    const int pw = (t_opaque >> 6) - 4;
    const int c0 = 4 * (pw * CQW + cql), i0 = tg * TPL;
    constexpr uint32_t kSign = 0x80000000u;
    uint32_t nG[TPL][4];
    float lmax = -1.f;    // largest per-token log2|alpha|: > 0 means a gate above 1
    {
      float mag[4] = {0.f, 0.f, 0.f, 0.f};
      uint32_t par[4] = {0u, 0u, 0u, 0u};
      if (nt_c < C) {     // padding tokens: identity gate, zero key and query
#pragma unroll
        for (int r = 0; r < TPL; ++r)
          if (i0 + r >= nt_c) {
            in_a[r] = make_float4(1.f, 1.f, 1.f, 1.f);
            in_k[r] = make_uint2(0u, 0u);
            in_q[r] = make_uint2(0u, 0u);
          }
      }
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const float a4[4] = {in_a[r].x, in_a[r].y, in_a[r].z, in_a[r].w};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float lg = fmaxf(flog2(fabsf(a4[cc])), kLog2Floor);
          lmax = fmaxf(lmax, lg);
          mag[cc] -= lg;
          if (SIGNED) par[cc] ^= __builtin_bit_cast(uint32_t, a4[cc]);
          // mag may be -0 (a lane of padding tokens): take its magnitude bits only
          nG[r][cc] = (par[cc] & kSign) | (__builtin_bit_cast(uint32_t, mag[cc]) & ~kSign);
        }
      }
    }
    // inclusive scan of the lane totals over the token groups (lanes CQW apart):
    // magnitudes add, parities xor
    uint32_t incl[4] = {nG[TPL - 1][0], nG[TPL - 1][1], nG[TPL - 1][2], nG[TPL - 1][3]};
#pragma unroll
    for (int d = 1; d < TGW; d <<= 1) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint32_t y = __shfl_up(incl[cc], d * CQW);
        if (tg >= d) {
          const float m = fabsf(__builtin_bit_cast(float, incl[cc])) + fabsf(__builtin_bit_cast(float, y));
          incl[cc] = (SIGNED ? ((incl[cc] ^ y) & kSign) : 0u) | __builtin_bit_cast(uint32_t, m);
        }
      }
    }
    float base[4];
    uint32_t exb[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint32_t y = __shfl_up(incl[cc], CQW);
      const uint32_t ex = tg ? y : 0u;
      const uint32_t tot = __shfl(incl[cc], (TGW - 1) * CQW + cql);
      const float half = 0.5f * fabsf(__builtin_bit_cast(float, tot));   // -R = -G_n / 2
      // D = G - R = half - (|ex| + |m|);  pre = 2^R, post = (-1)^pi_n 2^(G_n - R): same magnitude
      base[cc] = half - fabsf(__builtin_bit_cast(float, ex));
      exb[cc] = ex;
      const float e = fexp2(-half);
      pre4[cc] = e;
      post4[cc] = SIGNED ? __builtin_bit_cast(float, (tot & kSign) | __builtin_bit_cast(uint32_t, e)) : e;
    }
    // q/k normalisation factors (sum of squares + 1e-6)^(-1/2) per token
    float fk[TPL], fq[TPL];
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      fk[r] = 1.f;
      fq[r] = 1.f;
      if (NORM) {
        float sk = 1e-6f, sq = 1e-6f;
#pragma unroll
        for (int pw2 = 0; pw2 < 4; ++pw2) {
          const float2 pp = *reinterpret_cast<const float2 *>(s_nrm + (pw2 * C + i0 + r) * 2);
          sk += pp.x;
          sq += pp.y;
        }
        fk[r] = __builtin_amdgcn_rsqf(sk);
        fq[r] = __builtin_amdgcn_rsqf(sq);
        if (pw == 0 && cql == 0)
          *reinterpret_cast<float2 *>(s_fac + (i0 + r) * 2) = make_float2(fk[r], fq[r]);
      }
    }
    float gmax = 0.f;
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      float gk[4], gq[4], kg[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float D = base[cc] - fabsf(__builtin_bit_cast(float, nG[r][cc]));
        gmax = fmaxf(gmax, fabsf(D));
        const uint32_t sgn = SIGNED ? (nG[r][cc] ^ exb[cc]) & kSign : 0u;
        const float gam = __builtin_bit_cast(float, sgn | __builtin_bit_cast(uint32_t, fexp2(D)));
        const float igam = __builtin_bit_cast(float, sgn | __builtin_bit_cast(uint32_t, fexp2(-D)));
        const uint32_t kw = cc < 2 ? in_k[r].x : in_k[r].y, qw = cc < 2 ? in_q[r].x : in_q[r].y;
        float kk = __builtin_bit_cast(float, (cc & 1) ? (kw & 0xFFFF0000u) : (kw << 16));
        float qq = __builtin_bit_cast(float, (cc & 1) ? (qw & 0xFFFF0000u) : (qw << 16));
        if (NORM) {
          kk *= fk[r];
          qq *= fq[r];
        }
        gk[cc] = -kk * gam;
        gq[cc] = qq * gam;
        kg[cc] = kk * igam;
      }
      const int i = i0 + r;
      uint2 h, l;
      split_quad(gk, h, l);
      *reinterpret_cast<uint2 *>(gk_h + at(i, c0, DK)) = h;
      *reinterpret_cast<uint2 *>(gk_l + at(i, c0, DK)) = l;
      split_quad(gq, h, l);
      *reinterpret_cast<uint2 *>(gq_h + at(i, c0, DK)) = h;
      *reinterpret_cast<uint2 *>(gq_l + at(i, c0, DK)) = l;
      split_quad(kg, o_kg_h[r], o_kg_l[r]);
      __builtin_amdgcn_sched_barrier(0);   // one token at a time: bounded live range
    }
    // The factored ratios need |G - R| <= kGuard and a log-gate that never rises
    // (|alpha| <= 1, so -G >= 0 can share its word with the parity bit); any
    // other chunk takes the element-wise path.
    guard_bad = __any(gmax > kGuard || lmax > 0.f) ? 1u : 0u;
  };

  if (threadIdx.x == 0) { s_flag[0] = 0; s_flag[1] = 0; }

  // The two roles run separate loops with the same barrier sequence per chunk
  // (H1, H2, H3, two more on the exact path, H4), so each role's registers are
  // live only inside its own loop.
  if (prep) {
    // ======================= chunk preparation (waves 4-7)
    float xA[6];        // exact path: the off-diagonal -A blocks, held over one barrier
    if (nch > 0) {
      pr_load(0, threadIdx.x, 2);
      if (NORM) pr_partials(threadIdx.x);
    }
    __syncthreads();   // B0: the first chunk's norm partials
    if (nch > 0) pr_compute(min(C, len));
    for (int lc = 0; lc < nch; ++lc) {
      const int t0 = start + lc * C, nt = min(C, len - lc * C);
      int t_opaque = threadIdx.x;
      asm volatile("" : "+v"(t_opaque));
      const int lane = t_opaque & 63, l16 = lane & 15, gq = lane >> 4;
      const int tid = t_opaque - 256;                       // preparation thread
      const int pw = __builtin_amdgcn_readfirstlane(tid >> 6);   // preparation wave (uniform)
      const int tg = lane / CQW, cql = lane % CQW;
      const int c0 = 4 * (pw * CQW + cql), i0 = tg * TPL;

      __syncthreads();   // H1: the previous chunk's operands are no longer read
      // ---- hand-off: the register stage's operands into LDS
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const int i = i0 + r;
        *reinterpret_cast<uint2 *>(kg_h + at(i, c0, DK)) = o_kg_h[r];
        *reinterpret_cast<uint2 *>(kg_l + at(i, c0, DK)) = o_kg_l[r];
      }
      // (K/gamma)^T: channel rows, 4 tokens per 8-byte store
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int r4 = 0; r4 < TPL; r4 += 4) {
          uint32_t hw[2], lw[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = r4 + 2 * u;
            const int sh = 16 * (cc & 1);
            const uint32_t h0 = (cc < 2 ? o_kg_h[r].x : o_kg_h[r].y) >> sh;
            const uint32_t h1 = (cc < 2 ? o_kg_h[r + 1].x : o_kg_h[r + 1].y) >> sh;
            const uint32_t l0 = (cc < 2 ? o_kg_l[r].x : o_kg_l[r].y) >> sh;
            const uint32_t l1 = (cc < 2 ? o_kg_l[r + 1].x : o_kg_l[r + 1].y) >> sh;
            hw[u] = (h0 & 0xFFFFu) | (h1 << 16);
            lw[u] = (l0 & 0xFFFFu) | (l1 << 16);
          }
          *reinterpret_cast<uint2 *>(kt_h + at(c0 + cc, i0 + r4, C)) = make_uint2(hw[0], hw[1]);
          *reinterpret_cast<uint2 *>(kt_l + at(c0 + cc, i0 + r4, C)) = make_uint2(lw[0], lw[1]);
        }
      if (tg == 0) {
        *reinterpret_cast<float4 *>(s_pre + c0) = make_float4(pre4[0], pre4[1], pre4[2], pre4[3]);
        *reinterpret_cast<float4 *>(s_mid + c0) = make_float4(1.f, 1.f, 1.f, 1.f);
        *reinterpret_cast<float4 *>(s_post + c0) =
            make_float4(post4[0], post4[1], post4[2], post4[3]);
      }
      if (pw == 0) s_beta[lane] = lane < nt ? in_b : 0.f;
      if (guard_bad && lane == 0) atomicOr(&s_flag[lc & 1], 1);

      __syncthreads();   // H2
      const int fallback = s_flag[lc & 1];
      if (lc + 1 < nch) pr_load(lc + 1, t_opaque, 0);   // next chunk's gates, in flight meanwhile
      f32x4 pA[3], pP[3];                      // A and P tiles, held over H3
      if (!fallback) {
        // ---- A and P tiles (I, J), J <= I, computed transposed: the MFMA's row
        // operand is K/gamma' of block J, its column operand -(gamma' K) or
        // gamma' Q of block I, so lane (g, l) ends up with row 16 I + l and the
        // four consecutive columns 16 J + 4 g .. +3.  Each wave takes tiles that
        // share their column operand block I:
        //   wave 0: (3,0) (3,1) (3,2)   wave 1: (2,0) (2,1) (2,2)
        //   wave 2: (1,0) (1,1)         wave 3: (0,0) (3,3)
        // Tile 0's fragments of k block kb + 1 are read while kb's products run;
        // the other tiles' fragments of block kb are read at the start of its step,
        // ahead of that prefetch, so waiting for them never waits for it.
        const int I0 = 3 - pw;
        const bool has1 = pw <= 2, has2 = pw != 2, row2 = pw == 3;
        const int J2 = pw == 3 ? 3 : 2;
        bf16x8 ka_h[2], ka_l[2], rk_h[2], rk_l[2], rq_h[2], rq_l[2];
        auto ld = [&](int kb) {
          const int sl2 = kb & 1;
          ka_h[sl2] = frag32(kg_h, DK, l16, kb, gq);
          ka_l[sl2] = frag32(kg_l, DK, l16, kb, gq);
          rk_h[sl2] = frag32(gk_h, DK, 16 * I0 + l16, kb, gq);
          rk_l[sl2] = frag32(gk_l, DK, 16 * I0 + l16, kb, gq);
          rq_h[sl2] = frag32(gq_h, DK, 16 * I0 + l16, kb, gq);
          rq_l[sl2] = frag32(gq_l, DK, 16 * I0 + l16, kb, gq);
        };
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          pA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          pP[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        ld(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int sl2 = kb & 1;
          bf16x8 kb_h, kb_l, kc_h, kc_l, sk_h, sk_l, sq_h, sq_l;
          if (has1) {
            kb_h = frag32(kg_h, DK, 16 + l16, kb, gq);
            kb_l = frag32(kg_l, DK, 16 + l16, kb, gq);
          }
          if (has2) {
            kc_h = frag32(kg_h, DK, 16 * J2 + l16, kb, gq);
            kc_l = frag32(kg_l, DK, 16 * J2 + l16, kb, gq);
          }
          if (row2) {
            sk_h = frag32(gk_h, DK, 48 + l16, kb, gq);
            sk_l = frag32(gk_l, DK, 48 + l16, kb, gq);
            sq_h = frag32(gq_h, DK, 48 + l16, kb, gq);
            sq_l = frag32(gq_l, DK, 48 + l16, kb, gq);
          } else {
            sk_h = rk_h[sl2];
            sk_l = rk_l[sl2];
            sq_h = rq_h[sl2];
            sq_l = rq_l[sl2];
          }
          if (kb + 1 < KB) ld(kb + 1);
          __builtin_amdgcn_sched_barrier(0);
          pA[0] = mfma32x3(pA[0], ka_h[sl2], ka_l[sl2], rk_h[sl2], rk_l[sl2]);
          pP[0] = mfma32x3(pP[0], ka_h[sl2], ka_l[sl2], rq_h[sl2], rq_l[sl2]);
          if (has1) {
            pA[1] = mfma32x3(pA[1], kb_h, kb_l, rk_h[sl2], rk_l[sl2]);
            pP[1] = mfma32x3(pP[1], kb_h, kb_l, rq_h[sl2], rq_l[sl2]);
          }
          if (has2) {
            pA[2] = mfma32x3(pA[2], kc_h, kc_l, sk_h, sk_l);
            pP[2] = mfma32x3(pP[2], kc_h, kc_l, sq_h, sq_l);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // pA holds -A_ij / beta_i; scale by beta_i (row 16 I + l16) -> -A_ij.
        // Diagonal tiles also go to the fp32 store, transposed, zero on and above
        // the diagonal.
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          if (t == 0 || (t == 1 && has1) || (t == 2 && has2)) {
            const int I = (t == 2 && row2) ? 3 : I0, J = t == 2 ? J2 : t;
            const float bi = s_beta[16 * I + l16];
#pragma unroll
            for (int e = 0; e < 4; ++e) pA[t][e] *= bi;
            if (I == J) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                s_ad[I * ADB + (4 * gq + e) * ADS + l16] = 4 * gq + e < l16 ? -pA[t][e] : 0.f;
            }
          }
        }
      } else {
        // ---- exact path, part 1: G (fp32) per (token, channel) and the parity
        // mask of each channel into the K/gamma region, one channel per thread.
        float *s_G = reinterpret_cast<float *>(smem + L::KG);
        uint2 *s_pm = reinterpret_cast<uint2 *>(smem + L::KG + L::FG);   // [DK] 64-bit masks
        const int c = tid;
        if (c < DK) {
          float G = 0.f;
          uint32_t par = 0, m0 = 0, m1 = 0;
          for (int i = 0; i < C; ++i) {
            const float a = i < nt ? g[((size_t)(t0 + i) * H + h) * DK + c] : 1.f;
            G += fmaxf(flog2(fabsf(a)), kLog2Floor);
            if (SIGNED) par ^= a < 0.f ? 1u : 0u;
            s_G[i * DK + c] = G;
            if (i < 32) m0 |= par << i; else m1 |= par << (i - 32);
          }
          s_pm[c] = make_uint2(m0, m1);
        }
      }

      __syncthreads();   // H3
      if (lc + 1 < nch) pr_load(lc + 1, t_opaque, 1);   // and its keys, queries, beta
      if (!fallback) {
        // -A below the diagonal blocks, P on and below them: 8-byte stores
        const int I0 = 3 - pw;
        const bool has1 = pw <= 2, has2 = pw != 2, row2 = pw == 3;
        const int J2 = pw == 3 ? 3 : 2;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          if (t == 0 || (t == 1 && has1) || (t == 2 && has2)) {
            const int I = (t == 2 && row2) ? 3 : I0, J = t == 2 ? J2 : t;
            const int i = 16 * I + l16, j = 16 * J + 4 * gq;
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = (J < I || 4 * gq + e <= l16) ? pP[t][e] : 0.f;
            uint2 hh, ll;
            split_quad(pv, hh, ll);
            *reinterpret_cast<uint2 *>(p_h + at(i, j, C)) = hh;
            *reinterpret_cast<uint2 *>(p_l + at(i, j, C)) = ll;
            if (J < I) {
              const float av[4] = {pA[t][0], pA[t][1], pA[t][2], pA[t][3]};
              split_quad(av, hh, ll);
              *reinterpret_cast<uint2 *>(at_h + at(i, j, C)) = hh;
              *reinterpret_cast<uint2 *>(at_l + at(i, j, C)) = ll;
            }
          }
        }
        // P's blocks (0,1) and (2,3) are read by the 32-token P U products: zero them
        {
          const int blk2 = tid >> 7, e = (tid & 127) * 2;     // 2 blocks x 128 threads x 2
          const int i = 32 * blk2 + (e >> 4), j = 32 * blk2 + 16 + (e & 15);
          *reinterpret_cast<uint32_t *>(p_h + at(i, j, C)) = 0u;
          *reinterpret_cast<uint32_t *>(p_l + at(i, j, C)) = 0u;
        }
      } else {
        // ---- exact path, part 2: A and P element by element (fp32 ratios
        // 2^(G_i - G_j), whatever their size) into registers, the diagonal A tiles,
        // K_hat^T = (K gamma_n / gamma)^T and the operands relative to the chunk
        // start; the state pass then uses S_pre = S and
        // S' = Diag(gamma_n) S + K_hat^T U.
        const float *s_G = reinterpret_cast<const float *>(smem + L::KG);
        const uint2 *s_pm = reinterpret_cast<const uint2 *>(smem + L::KG + L::FG);
        auto par_of = [&](int i, int c) {
          const uint2 m = s_pm[c];
          return ((i < 32 ? m.x : m.y) >> (i & 31)) & 1u;
        };
        // one (i, j) element per thread and step; returns sum_c k_i,c r_ij,c x_j,c
        // for x = k (A) and the query's row for P
        auto exact_pair = [&](int i, int j, float &accA, float &accP) {
          accA = 0.f;
          accP = 0.f;
          if (j <= i && i < nt) {
            const size_t ri = (size_t)(t0 + i) * H + h, rj = (size_t)(t0 + j) * H + h;
            for (int c = 0; c < DK; ++c) {
              const float r = with_sign(fexp2(s_G[i * DK + c] - s_G[j * DK + c]),
                                        par_of(i, c) ^ par_of(j, c));
              const float kj = __bfloat162float(k[rj * DK + c]) * r;
              accA += __bfloat162float(k[ri * DK + c]) * kj;
              accP += __bfloat162float(q[ri * DK + c]) * kj;
            }
            if (NORM) {
              accA *= s_fac[2 * i] * s_fac[2 * j];
              accP *= s_fac[2 * i + 1] * s_fac[2 * j];
            }
          }
        };
        // P (all of it, zero above the diagonal) and the diagonal A tiles go
        // straight to LDS; the six off-diagonal -A blocks wait in registers
        // until the G table is dead.
        for (int u = 0; u < (C * C) / 256; ++u) {
          const int pp = tid + 256 * u, i = pp / C, j = pp % C;
          float accA, accP;
          exact_pair(i, j, accA, accP);
          __bf16 hh, ll;
          split1(accP, hh, ll);
          p_h[at(i, j, C)] = hh;
          p_l[at(i, j, C)] = ll;
          if ((i >> 4) == (j >> 4))
            s_ad[(i >> 4) * ADB + (j & 15) * ADS + (i & 15)] = (j < i) ? s_beta[i] * accA : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          int I, J;
          tile_of_pair(u < 1 ? 1 : u < 3 ? u + 2 : u + 3, I, J);   // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
          const int i = 16 * I + (tid >> 4), j = 16 * J + (tid & 15);
          float accA, accP;
          exact_pair(i, j, accA, accP);
          xA[u] = -s_beta[i] * accA;
        }
        for (int pp = tid; pp < DK * C; pp += 256) {
          const int c = pp / C, j = pp % C;
          float x = 0.f;
          if (j < nt) {
            const float r = with_sign(fexp2(s_G[(C - 1) * DK + c] - s_G[j * DK + c]),
                                      par_of(C - 1, c) ^ par_of(j, c));
            x = __bfloat162float(k[((size_t)(t0 + j) * H + h) * DK + c]) * r;
            if (NORM) x *= s_fac[2 * j];
          }
          __bf16 hh, ll;
          split1(x, hh, ll);
          kt_h[at(c, j, C)] = hh;
          kt_l[at(c, j, C)] = ll;
        }
        // -(gamma K) and gamma Q relative to the chunk start
        for (int pp = tid; pp < C * DK; pp += 256) {
          const int i = pp / DK, c = pp % DK;
          float xk = 0.f, xq = 0.f;
          if (i < nt) {
            const float gam = with_sign(fexp2(s_G[i * DK + c]), par_of(i, c));
            const size_t ri = (size_t)(t0 + i) * H + h;
            xk = -__bfloat162float(k[ri * DK + c]) * gam;
            xq = __bfloat162float(q[ri * DK + c]) * gam;
            if (NORM) {
              xk *= s_fac[2 * i];
              xq *= s_fac[2 * i + 1];
            }
          }
          __bf16 hh, ll;
          split1(xk, hh, ll);
          gk_h[at(i, c, DK)] = hh;
          gk_l[at(i, c, DK)] = ll;
          split1(xq, hh, ll);
          gq_h[at(i, c, DK)] = hh;
          gq_l[at(i, c, DK)] = ll;
        }
        for (int c = tid; c < DK; c += 256) {
          s_pre[c] = 1.f;
          s_mid[c] = with_sign(fexp2(s_G[(C - 1) * DK + c]), par_of(C - 1, c));
          s_post[c] = 1.f;
        }
        __syncthreads();   // every thread is done reading G: its region takes -A
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          int I, J;
          tile_of_pair(u < 1 ? 1 : u < 3 ? u + 2 : u + 3, I, J);
          const int i = 16 * I + (tid >> 4), j = 16 * J + (tid & 15);
          __bf16 hh, ll;
          split1(xA[u], hh, ll);
          at_h[at(i, j, C)] = hh;
          at_l[at(i, j, C)] = ll;
        }
        __syncthreads();   // diagonal A tiles complete for the inverses
      }
      if (NORM && lc + 1 < nch) pr_partials(t_opaque);   // next chunk's keys and queries
      __syncthreads();   // H4
      if (lc + 1 < nch) pr_compute(min(C, len - (lc + 1) * C));   // overlaps the state pass
    }
  } else {
    // ======================= state pass (waves 0-3)
    {
      const int lane = threadIdx.x & 63, l16 = lane & 15, gq = lane >> 4;
      const int col = vb * BV + 16 * w + l16;
#pragma unroll
      for (int tt = 0; tt < ST; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accS[tt][e] =
              S0 ? S0[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] : 0.f;
      if (nch > 0) sp_load_v(0, threadIdx.x);
    }
    __syncthreads();   // B0
    for (int lc = 0; lc < nch; ++lc) {
      const int t0 = start + lc * C, nt = min(C, len - lc * C);
      int t_opaque = threadIdx.x;
      asm volatile("" : "+v"(t_opaque));
      const int lane = t_opaque & 63, l16 = lane & 15, gq = lane >> 4;
      const int col = vb * BV + 16 * (t_opaque >> 6) + l16;
      // per-lane LDS byte offsets of the regions this loop reads
      const int lpD = pb(l16, 4 * gq, DK), lpC = pb(l16, 4 * gq, C);
      const int gk_b = opaque(L::GK + lpD), gq_b = opaque(L::GQ + lpD);
      const int kt_b = opaque(L::KT + lpC), p_b = opaque(L::P + lpC);
      const int at_b = opaque(L::AT + lpC), fac_b = opaque(L::SPRE + 16 * gq);
      const int bt_b = opaque(L::BT + 16 * gq);
      constexpr int LO_D = 2 * C * (DK + PADB), LO_C = 2 * C * (C + PADB);
      constexpr int LO_T = 2 * DK * (C + PADB);

      __syncthreads();   // H1
      if (threadIdx.x == 0) s_flag[(lc + 1) & 1] = 0;
      __syncthreads();   // H2
      const int fallback = s_flag[lc & 1];

      // ---- S_pre = pre * S;  X = V - (gamma' K) S_pre;  O = (gamma' Q) S_pre
      f32x4 accX[4], accO[4];
      auto x_and_o = [&]() {
#pragma unroll
        for (int tt = 0; tt < ST; ++tt) {
          const float4 pre = lds_at<float4>(smem, fac_b, 64 * tt);
          accS[tt][0] *= pre.x; accS[tt][1] *= pre.y; accS[tt][2] *= pre.z; accS[tt][3] *= pre.w;
        }
        bf16x8 sh[KB], sl[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) split8_acc(accS[2 * kb], accS[2 * kb + 1], sh[kb], sl[kb]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            accX[mt][e] = 16 * mt + 4 * gq + e < nt ? bf16_to_f32(in_v[mt][e]) : 0.f;
          accO[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // 4 KB steps (mt, kb); the row fragments of step st + 2 are read while
        // step st's products run (a ring of three register slots)
        constexpr int NS = 4 * KB;
        bf16x8 rk_h[3], rk_l[3], rq_h[3], rq_l[3];
        auto ld = [&](int st) {
          const int mt = st / KB, kb = st % KB, sl3 = st % 3;
          rk_h[sl3] = frag32o(smem, gk_b, pb(16 * mt, 32 * kb, DK));
          rk_l[sl3] = frag32o(smem, gk_b, LO_D + pb(16 * mt, 32 * kb, DK));
          rq_h[sl3] = frag32o(smem, gq_b, pb(16 * mt, 32 * kb, DK));
          rq_l[sl3] = frag32o(smem, gq_b, LO_D + pb(16 * mt, 32 * kb, DK));
        };
        ld(0);
        ld(1);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          if (st + 2 < NS) ld(st + 2);
          __builtin_amdgcn_sched_barrier(0);
          const int mt = st / KB, kb = st % KB, sl3 = st % 3;
          accX[mt] = mfma32x3(accX[mt], rk_h[sl3], rk_l[sl3], sh[kb], sl[kb]);
          accO[mt] = mfma32x3(accO[mt], rq_h[sl3], rq_l[sl3], sh[kb], sl[kb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (lc + 1 < nch) sp_load_v(lc + 1, t_opaque);
      };
      if (!fallback) x_and_o();

      __syncthreads();   // H3
      if (fallback) {    // the exact path rewrites the operands first
        __syncthreads();
        __syncthreads();
        x_and_o();
      }
      if ((t_opaque >> 6) == 0) {
        // (I + A_II)^-1 for the four diagonal blocks, column j of block I per lane,
        // by right-looking forward substitution: once x_m is final it is
        // subtracted from every later row.  A_II is stored transposed, so the
        // entries below x_m are one row of the store, read four at a time; no
        // read depends on x, so all of them can be in flight early.
        const int I = lane >> 4, j = lane & 15;
        const int ad_b = opaque(L::AD + 4 * I * ADB);
        const int ti_b = opaque(L::AT + pb(16 * I, 16 * I + j, C));
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
          float4 r[4];
#pragma unroll
          for (int q4 = (m + 1) / 4; q4 < 4; ++q4)
            r[q4] = lds_at<float4>(smem, ad_b, 4 * (m * ADS + 4 * q4));
#pragma unroll
          for (int i = m + 1; i < 16; ++i) {
            const float4 &rq = r[i / 4];
            const float a = (i & 3) == 0 ? rq.x : (i & 3) == 1 ? rq.y : (i & 3) == 2 ? rq.z : rq.w;
            x[i] -= a * x[m];
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __bf16 hh, ll;
          split1(x[i], hh, ll);
          *reinterpret_cast<__bf16 *>(smem + ti_b + pb(i, 0, C)) = hh;
          *reinterpret_cast<__bf16 *>(smem + ti_b + LO_C + pb(i, 0, C)) = ll;
        }
      }
      __syncthreads();   // H4

      // ---- (I + A) U = Diag(beta) X by block forward substitution.  U's hi/lo
      // parts are kept per 16-token block (the B operand of a 16x16x16 product);
      // two consecutive blocks side by side form the 32-token B operand in the
      // accumulator k order of the 16x16x32 products.  All of the solve's row
      // fragments are read up front.
      bf16x4 dh[4], dl[4], b1h, b1l, b3h, b3l;
      bf16x8 c2h, c2l, c3h, c3l;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        dh[I] = frag16o(smem, at_b, pb(16 * I, 16 * I, C));
        dl[I] = frag16o(smem, at_b, LO_C + pb(16 * I, 16 * I, C));
      }
      b1h = frag16o(smem, at_b, pb(16, 0, C));
      b1l = frag16o(smem, at_b, LO_C + pb(16, 0, C));
      c2h = frag32o(smem, at_b, pb(32, 0, C));
      c2l = frag32o(smem, at_b, LO_C + pb(32, 0, C));
      c3h = frag32o(smem, at_b, pb(48, 0, C));
      c3l = frag32o(smem, at_b, LO_C + pb(48, 0, C));
      b3h = frag16o(smem, at_b, pb(48, 32, C));
      b3l = frag16o(smem, at_b, LO_C + pb(48, 32, C));
      bf16x4 uh[4], ul[4];
      auto u32h = [&](int kb) { return __builtin_shufflevector(uh[2 * kb], uh[2 * kb + 1], 0, 1, 2, 3, 4, 5, 6, 7); };
      auto u32l = [&](int kb) { return __builtin_shufflevector(ul[2 * kb], ul[2 * kb + 1], 0, 1, 2, 3, 4, 5, 6, 7); };
      // P fragments for the first two O += P U steps, read during the solve
      constexpr int kPuMt[6] = {0, 1, 2, 2, 3, 3}, kPuKb[6] = {0, 0, 0, 1, 0, 1};
      bf16x8 rp_h[3], rp_l[3];
      auto ldp = [&](int st) {
        rp_h[st % 3] = frag32o(smem, p_b, pb(16 * kPuMt[st], 32 * kPuKb[st], C));
        rp_l[st % 3] = frag32o(smem, p_b, LO_C + pb(16 * kPuMt[st], 32 * kPuKb[st], C));
      };
      ldp(0);
      ldp(1);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 y;
        const float4 bq = lds_at<float4>(smem, bt_b, 64 * I);
        y[0] = bq.x * accX[I][0];
        y[1] = bq.y * accX[I][1];
        y[2] = bq.z * accX[I][2];
        y[3] = bq.w * accX[I][3];
        if (I == 1) y = mfma16x3(y, b1h, b1l, uh[0], ul[0]);
        if (I == 2) y = mfma32x3(y, c2h, c2l, u32h(0), u32l(0));
        if (I == 3) {
          y = mfma32x3(y, c3h, c3l, u32h(0), u32l(0));
          y = mfma16x3(y, b3h, b3l, uh[2], ul[2]);
        }
        if (I == 1 || I == 3) settle16();
        bf16x4 yh, yl;
        split4(y, yh, yl);
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        u = mfma16x3(u, dh[I], dl[I], yh, yl);
        settle16();
        split4(u, uh[I], ul[I]);
      }
      // ---- O += P U (P is zero above its diagonal blocks); store
#pragma unroll
      for (int st = 0; st < 6; ++st) {
        if (st + 2 < 6) ldp(st + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int mt = kPuMt[st], kb = kPuKb[st];
        accO[mt] = mfma32x3(accO[mt], rp_h[st % 3], rp_l[st % 3], u32h(kb), u32l(kb));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (OBF16) {
        const int rs = H * DV * 2;
        const auto ro = rsrc(static_cast<__hip_bfloat16 *>(o) + ((size_t)t0 * H + h) * DV,
                             (nt - 1) * rs + DV * 2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float val = accO[mt][e];
            asm volatile("v_mov_b32 %0, %1" : "=v"(val) : "v"(val));
            const __bf16 b = (__bf16)val;
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, b), ro,
                                                  (16 * mt + 4 * gq + e) * rs + 2 * col, 0, 0);
          }
      } else {
        const int rs = H * DV * 4;
        const auto ro = rsrc(static_cast<float *>(o) + ((size_t)t0 * H + h) * DV, (nt - 1) * rs + DV * 4);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // A store reads its data register after issue, so the accumulator it
            // came from could not be reused until the write completed; store a
            // copy instead (this also reads the vector element through a scalar,
            // as a bit_cast of the element itself took element 0).
            float val = accO[mt][e];
            asm volatile("v_mov_b32 %0, %1" : "=v"(val) : "v"(val));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), ro,
                                                  (16 * mt + 4 * gq + e) * rs + 4 * col, 0, 0);
          }
      }
      // ---- S <- post * (mid * S_pre + (KT plane)^T U): 2 ST steps (tile, kb),
      // fragments read two steps ahead
      {
        constexpr int NS = 2 * ST;
        bf16x8 rt_h[3], rt_l[3];
        auto ld = [&](int st) {
          const int tt = st >> 1, kb = st & 1, sl3 = st % 3;
          rt_h[sl3] = frag32o(smem, kt_b, pb(16 * tt, 32 * kb, C));
          rt_l[sl3] = frag32o(smem, kt_b, LO_T + pb(16 * tt, 32 * kb, C));
        };
        ld(0);
        ld(1);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          if (st + 2 < NS) ld(st + 2);
          __builtin_amdgcn_sched_barrier(0);
          const int tt = st >> 1, kb = st & 1, sl3 = st % 3;
          if (kb == 0) {
            if (fallback) {   // the mid factor is 1 except on the element-wise path
              const float4 mid = lds_at<float4>(smem, fac_b, (L::SMID - L::SPRE) + 64 * tt);
              accS[tt][0] *= mid.x; accS[tt][1] *= mid.y; accS[tt][2] *= mid.z; accS[tt][3] *= mid.w;
            }
          }
          accS[tt] = mfma32x3(accS[tt], rt_h[sl3], rt_l[sl3], u32h(kb), u32l(kb));
          if (kb == 1) {
            const float4 post = lds_at<float4>(smem, fac_b, (L::SPOST - L::SPRE) + 64 * tt);
            accS[tt][0] *= post.x; accS[tt][1] *= post.y; accS[tt][2] *= post.z; accS[tt][3] *= post.w;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if (!prep && S_T) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, gq = lane >> 4;
    const int col = vb * BV + 16 * w + l16;
#pragma unroll
    for (int tt = 0; tt < ST; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_T[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] = accS[tt][e];
  }
}

template <int DK, bool SIGNED, bool NORM, bool OBF16>
hipError_t launch_dk(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                     int DV, int N, SeqTable tab, int packed, hipStream_t stream) {
  const int NH = N * H, NV = DV / BV;
  const int groups = (NH + 7) / 8;
  const dim3 grid((unsigned)groups * 8u * (unsigned)NV), block(NT);
  hipLaunchKernelGGL((fwd_bf16_kernel<DK, SIGNED, NORM, OBF16>), grid, block, 0, stream,
                     static_cast<const __hip_bfloat16 *>(q), static_cast<const __hip_bfloat16 *>(k),
                     static_cast<const __hip_bfloat16 *>(v), g, beta, S0, o, S_T, T, H, DV, NH, NV,
                     tab, packed);
  return hipGetLastError();
}

// One kernel per option combination, so no option costs a branch in the loop.
template <int DK>
hipError_t launch_opts(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                       int DV, int N, SeqTable tab, int packed, int signed_gates, int l2norm,
                       int o_bf16, hipStream_t stream) {
#define CKDA_BF16_CASE(S_, N_, O_)                                                             \
  if (!!signed_gates == S_ && !!l2norm == N_ && !!o_bf16 == O_)                                \
    return launch_dk<DK, S_, N_, O_>(q, k, v, g, beta, S0, o, S_T, T, H, DV, N, tab, packed,  \
                                     stream);
  CKDA_BF16_CASE(true, false, false)
  CKDA_BF16_CASE(false, false, false)
  CKDA_BF16_CASE(true, true, false)
  CKDA_BF16_CASE(false, true, false)
  CKDA_BF16_CASE(true, false, true)
  CKDA_BF16_CASE(false, false, true)
  CKDA_BF16_CASE(true, true, true)
  CKDA_BF16_CASE(false, true, true)
#undef CKDA_BF16_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                           int dk, int dv, int N, SeqTable tab, int packed, int signed_gates,
                           int l2norm, int o_bf16, hipStream_t stream) {
  if (dk == 64)
    return launch_opts<64>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, packed, signed_gates,
                           l2norm, o_bf16, stream);
  if (dk == 128)
    return launch_opts<128>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, packed, signed_gates,
                            l2norm, o_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace ckda
