// Fused chunkwise CKDA forward for bf16 q/k/v on CDNA4 matrix cores.
//
// One workgroup owns one (sequence, head, 64-column block of dv).  Its slice
// of the fp32 state (dk x 64) lives in MFMA accumulators for the whole
// sequence; q/k/alpha are read once per workgroup (the dv blocks of a head
// share them through the L2 of their XCD), v and o once.
//
// The sequence is walked in blocks of CB = 16 tokens.  Block algebra (update
// rule: blog post "One update, one quarter turn", ELI5 "The mirror", unrolled
// over a block with incoming state S; gamma_i is the product of the block's
// gates up to token i, per key channel):
//   A_ij = beta_i sum_c (gamma_ic k_ic) (k_jc / gamma_jc)      (i > j)
//   P_ij =        sum_c (gamma_ic q_ic) (k_jc / gamma_jc)      (j <= i)
//   X    = V - (gamma K) S,   U = (I + A)^-1 Diag(beta) X
//   O    = (gamma Q) S + P U
//   S'   = Diag(gamma_n) S + (K gamma_n / gamma)^T U
//
// Signed gates.  Only ratios of gammas matter, so each channel is referenced
// to the block's last token: gamma' = gamma / gamma_n = 1 / (product of the
// gates after the token), formed as a running product of the signed gates
// (each gate's magnitude floored at 2^-126), so the sign needs no separate
// bookkeeping.  While every gamma' and 1/gamma' of the block lies within
// 2^+-110 (gates averaging above 2^-6.8 in magnitude over 16 tokens), A and P
// are one matrix-core product each of gamma'-scaled operands, and the state
// absorbs gamma_n once per block:
//   S_pre = Diag(gamma_n) S,  X = V - (gamma' K) S_pre,  O = (gamma' Q) S_pre + P U,
//   S' = S_pre + (K / gamma')^T U.
// A block whose spread is wider takes an exact path that works in log space,
// as the CKDA summary ("Methodology in Plain English") keeps gate magnitudes:
// per channel the cumulative sum G of log2|alpha| (each term floored at -126)
// and the cumulative parity of negative gates.  A and P come from two
// matrix-core passes with half-block references (each ratio split about the
// last token of its column's half, so inside a half it is the factored form of
// an eight-token block, and across the halves both factors are products of
// gates); a half whose own spread exceeds 2^110 sends the block to A and P
// element by element from fp32 ratios 2^(G_i - G_j).  Either way the state
// pass's operands are referenced to the block start (X = V - (gamma K) S),
// S' = Diag(gamma_n) S + (K gamma_n / gamma)^T U.
//
// Work split inside the workgroup (512 threads), a pipeline with no barrier
// inside the sequence loop:
//   waves 4-7  preparation: wave 4 + b prepares block b of every 64-token
//              round (gate products, gamma'-scaled operands and their hi/lo bf16
//              split, A and P on matrix cores, (I + A)^-1 by substitution, a
//              row per quad of lanes) into LDS slot b;
//   waves 0-3  state pass, 16 dv columns each: X, O, U and the state update
//              on matrix cores, slot after slot.
// Two LDS counters per slot hand it over: `ready` (the slot holds round r's
// block) and `done` (all four state waves have finished reading it), so each
// preparation wave refills its slot for round r + 1 while the state pass works
// through the other three.  Every wait is bounded (kSpinLimit polls).
//
// Precision: every contraction whose operands are not raw bf16 inputs splits
// each fp32 operand x into hi = bf16(x) and lo = bf16(x - hi) and accumulates
// hi*hi + hi*lo + lo*hi in fp32, keeping ~16 mantissa bits: three MFMAs over
// 32 channels, or two over 16 tokens (both halves of a 32-deep product used).
//
// MFMA shape, 16x16x32 only (lane l, g = l / 16): A row l%16 / B column l%16
// hold k = 8g .. 8g+7; C rows 4g .. 4g+3.  An accumulator pair used as a B
// operand supplies k rows {4g..4g+3, 16+4g..16+4g+3}; the matching A operand
// is read in that order.  Over 16 tokens, lane g's k slots are tokens 4g ..
// 4g+3 twice: once against the hi operand, once against the lo one.
#include "ckda_internal.h"

namespace ckda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


constexpr int C = kChunk;        // tokens per round of the four preparation waves
constexpr int CB = 16;           // tokens per block
constexpr int NB = C / CB;       // block slots, one preparation wave each
constexpr int NT = 512;          // 8 waves per workgroup
constexpr int BV = 64;           // dv columns per workgroup (16 per state-pass wave)
constexpr int ADS = 20;          // row stride of the fp32 A tile (16-byte rows)
constexpr float kLog2Floor = -126.f;
constexpr float kGuardScale = 0x1p110f;   // bound on gamma_n / gamma_t and its inverse
constexpr float kGateFloor = 0x1p-126f;    // floor of a gate's magnitude
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: raw 32-bit data
constexpr int kSpinLimit = 1 << 18;        // polls of a hand-over counter before giving up
template <bool B>
struct Kind {                    // compile-time block kind (true: exact)
  static constexpr bool value = B;
};
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

template <class T>
__device__ __forceinline__ T lds_at(const char *smem, int base, int imm) {
  return *reinterpret_cast<const T *>(smem + base + imm);
}
// 16x16x32 fragment stored contiguously (16 bytes at base + imm, 16-byte aligned)
__device__ __forceinline__ bf16x8 frag32p(const char *smem, int base, int imm) {
  return __builtin_bit_cast(bf16x8, lds_at<uint4>(smem, base, imm));
}
// a fragment unit as the 16x16x32 operand [hi | lo]
__device__ __forceinline__ bf16x8 as_frag8(const uint4 &w) { return __builtin_bit_cast(bf16x8, w); }
__device__ __forceinline__ bf16x8 cat8(const bf16x4 &a, const bf16x4 &b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// v from lane s of each quad of lanes (s constant after unrolling)
__device__ __forceinline__ float quad_bcast(float v, int s) {
  const int x = __builtin_bit_cast(int, v);
  switch (s) {
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, false));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, false));
  }
}

// ---------------------------------------------------------------- LDS layout
// One slot per block position b (0..3): everything the state pass reads for a
// block, plus the preparation wave's own scratch.  bf16 planes are hi then lo.
// [CB][DK] rows are padded by 16 bytes and their channels permuted within each
// 32-channel block, so a lane's 16x16x32 fragment is one aligned 16-byte read.
// (K / gamma')^T, T and P are kept in fragment order: one 16-byte unit per
// (16-row tile, lane (l16, g)), the four hi bf16 of row l16, columns 4g .. 4g+3,
// then the four lo ones.  Read whole, a unit is the 16x16x32 operand [hi | lo]:
// against [b_hi | b_hi] it gives hi b_hi + lo b_hi, against [b_lo | 0] hi b_lo.
template <int DK>
struct Slot {
  static constexpr int RW = DK + 8;             // row of a [CB][DK] plane (elements, 16-byte rows)
  static constexpr int PL = CB * RW * 2;        // bytes of one half of such a plane
  static constexpr int KTS = 16 * 129 * (DK / 32);   // bytes of the (K / gamma')^T fragments
  static constexpr int TU = 64 * 16;            // bytes of a 16 x 16 tile in fragment units
  static constexpr int GK = 0;                  // -(gamma' K)        [CB][DK]
  static constexpr int GQ = GK + 2 * PL;        // gamma' Q           [CB][DK]
  static constexpr int KG = GQ + 2 * PL;        // K / gamma'         [CB][DK] (preparation only)
  static constexpr int KT = KG + 2 * PL;        // (K / gamma')^T     16-byte units (kt_unit)
  static constexpr int TT = KT + KTS;           // T = (I + A)^-1     fragment units
  static constexpr int PT = TT + TU;            // P, zero above the diagonal, fragment units
  static constexpr int AD = PT + TU;            // A fp32 [CB][ADS], zero on and above the
                                                // diagonal (preparation only)
  static constexpr int PRE = AD + CB * ADS * 4; // gamma_n [DK], signed
  static constexpr int BT = PRE + DK * 4;       // beta [CB]
  static constexpr int MODE = BT + CB * 4;      // 0: factored, 1: exact
  static constexpr int NF = MODE + 16;          // q/k normalisation factors [CB][2]
                                                // (preparation only)
  static constexpr int SIZE = NF + CB * 8;
  // Exact path scratch: G fp32 [CB][DK] and the parity words in the K/gamma'
  // region; the raw (normalised) keys and queries, fp32 [CB][DK], in the GK and
  // GQ regions until the operands overwrite them.
  static constexpr int XG = KG;
  static constexpr int XP = KG + CB * DK * 4;
  static_assert(CB * DK * 4 + 64 * 4 <= 2 * PL, "exact-path tables fit the K/gamma' region");
  static_assert(SIZE % 16 == 0 && XG % 16 == 0 && GQ % 16 == 0, "16-byte alignment");
  // exact blocks: a [CB][DK] column plane in the (K / gamma')^T and T regions
  static_assert(KT + 2 * PL <= PT && KT % 16 == 0, "column plane below the P tile");
};

template <int DK>
struct PrepGeom {                 // preparation lanes: 8 channels x TPL tokens each
  static constexpr int CG = DK / 8;       // channel groups
  static constexpr int TG = 64 / CG;      // token groups
  static constexpr int TPL = CB / TG;     // tokens per lane
  static_assert(TG * TPL == CB && (TPL == 2 || TPL == 4) && CG % 4 == 0, "preparation geometry");
  // Channel group cg holds channels base .. base+3 (cc = 0..3) and base+16 ..
  // base+19 (cc = 4..7), base = 32 (cg / 4) + 4 (cg % 4): the eight are one
  // 16-byte run of the permuted [CB][DK] planes.
  static __device__ __forceinline__ int base(int cg) { return 32 * (cg / 4) + 4 * (cg % 4); }
  static __device__ __forceinline__ int chan(int cg, int cc) {
    return base(cg) + (cc & 3) + 16 * (cc >> 2);
  }
  static __device__ __forceinline__ int group_of(int c) { return 4 * (c / 32) + (c % 16) / 4; }
  static __device__ __forceinline__ int index_of(int c) { return 4 * ((c % 32) / 16) + c % 4; }
};

// Unit of (16-channel tile tt, lane group g, row l16) among the (K / gamma')^T
// fragments.  Tiles go in pairs of 128 units plus one unit of padding: a
// state-pass lane group reads sixteen consecutive units, and the sixteen
// preparation lanes that store one channel slot each (channel 32a + 4m + i,
// a, m = 0..3) reach units a + 4m + const modulo 16, all in different banks.
__device__ __forceinline__ int kt_unit(int tt, int g, int l16) {
  return 129 * (tt >> 1) + 64 * (tt & 1) + 16 * g + l16;
}

// Hand-over counters in LDS.  Every lane of a wave reads the same word, so the
// polling loop is uniform; it gives up after kSpinLimit polls, so a wait can
// never hang the workgroup.
__device__ __forceinline__ void wait_for(const int *ctr, int target) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const int v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(v) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
// Waits until the wave's LDS reads and writes are complete, then (one lane)
// raises the counter.
__device__ __forceinline__ void lds_quiesce() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void publish(int *ctr, int value, bool leader) {
  lds_quiesce();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (leader) __hip_atomic_store(ctr, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void count_done(int *ctr, bool leader) {
  lds_quiesce();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (leader) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <class T>
__device__ __forceinline__ void lds_put(char *smem, int off, T v) {
  *reinterpret_cast<T *>(smem + off) = v;
}
// element cc (0..7) of eight packed bf16 as fp32
__device__ __forceinline__ float bf16_of(const uint4 &w, int cc) {
  const uint32_t x = cc < 2 ? w.x : cc < 4 ? w.y : cc < 6 ? w.z : w.w;
  return __builtin_bit_cast(float, (cc & 1) ? (x & 0xFFFF0000u) : (x << 16));
}

// Exact path for one block: A and P element by element from fp32 ratios
// 2^(G_i - G_j) (signs from the parity words), with the G table and parity
// words the caller left in slot `sb`, the keys and queries read from global
// memory through the block's buffer resources (row stride `rsk` bytes) and,
// with NORM, the per-token factors in the slot's normalisation table.
// Lane -> row i = lane / 4, columns 4 (lane % 4) .. +3; `bi` is beta of row i.
template <int DK, bool SIGNED, bool NORM>
__device__ __forceinline__ void exact_tiles(char *smem, int sb, int lane, float bi,
                                            __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rq,
                                            int rsk) {
  using SL = Slot<DK>;
  constexpr int CG = PrepGeom<DK>::CG, TPL = PrepGeom<DK>::TPL;
  const int ii = lane >> 2, jq = lane & 3;
  const float *xg = reinterpret_cast<const float *>(smem + sb + SL::XG);
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(smem + sb + SL::XP);
  const float *xf = reinterpret_cast<const float *>(smem + sb + SL::NF);   // [CB][2] factors
  auto par1 = [&](int t, int c) {    // parity of (t, c)
    using PG = PrepGeom<DK>;
    return (xp[(t / TPL) * CG + PG::group_of(c)] >> ((t % TPL) * 8 + PG::index_of(c))) & 1u;
  };
  auto bf = [](unsigned short x) { return __builtin_bit_cast(float, (uint32_t)x << 16); };
  float accA[4] = {0.f, 0.f, 0.f, 0.f}, accP[4] = {0.f, 0.f, 0.f, 0.f};
  // one channel per step: few registers, since this runs beside the caller's state
#pragma unroll 1
  for (int c = 0; c < DK; ++c) {
    const float gi = xg[ii * DK + c];
    const float ki = bf(__builtin_amdgcn_raw_buffer_load_b16(rk, ii * rsk + 2 * c, 0, 0));
    const float qi = bf(__builtin_amdgcn_raw_buffer_load_b16(rq, ii * rsk + 2 * c, 0, 0));
    const uint32_t pi = SIGNED ? par1(ii, c) : 0u;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * jq + jj;
      const float kj = bf(__builtin_amdgcn_raw_buffer_load_b16(rk, j * rsk + 2 * c, 0, 0));
      const uint32_t odd = SIGNED ? pi ^ par1(j, c) : 0u;
      const float x = kj * with_sign(fexp2(gi - xg[j * DK + c]), odd) * (NORM ? xf[2 * j] : 1.f);
      accA[jj] += ki * x;
      accP[jj] += qi * x;
    }
  }
  const float fki = NORM ? xf[2 * ii] : 1.f, fqi = NORM ? xf[2 * ii + 1] : 1.f;
  float av[4], pv[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = 4 * jq + jj;
    av[jj] = j < ii ? bi * fki * accA[jj] : 0.f;
    pv[jj] = j <= ii ? fqi * accP[jj] : 0.f;
  }
  lds_put(smem, sb + SL::AD + 4 * (ii * ADS + 4 * jq), make_float4(av[0], av[1], av[2], av[3]));
  uint2 hh, ll;
  split_quad(pv, hh, ll);
  lds_put(smem, sb + SL::PT + 16 * (16 * jq + ii), make_uint4(hh.x, hh.y, ll.x, ll.y));
}

// ---------------------------------------------------------------- kernel
// SIGNED: CKDA (false: KDA mode, gate signs ignored).  NORM: q and k are
// L2-normalised per (token, head) on the fly.  OBF16: o is written as bf16.
// PIPE: 0, the fused kernel; 1 and 2, the two halves of the two-kernel
// hand-off it replaced (uniform rows only), kept for measurement: 1 runs only
// the preparation, one workgroup of four preparation waves per (sequence,
// head, 64-token round), and writes each prepared block's slot image to `img`;
// 2 runs the state pass with waves 4-7 loading those images into the slots.
template <int DK, bool SIGNED, bool NORM, bool OBF16, int PIPE>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_kernel(
    const __hip_bfloat16 *__restrict__ q, const __hip_bfloat16 *__restrict__ k,
    const __hip_bfloat16 *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const float *S0, void *__restrict__ o,
    float *S_T, int T, int H, int DV, int NH, int NV, SeqTable tab, int packed,
    char *__restrict__ img) {
  using SL = Slot<DK>;
  using PG = PrepGeom<DK>;
  constexpr int CG = PG::CG, TG = PG::TG, TPL = PG::TPL;
  constexpr int KB = DK / 32;     // 32-channel k blocks
  constexpr int ST = DK / 16;     // 16-row state tiles per state-pass wave
  constexpr int SLOT = SL::SIZE;
  __shared__ __align__(16) char smem[NB * SLOT + 2 * NB * 4];
  int *s_ready = reinterpret_cast<int *>(smem + NB * SLOT);
  int *s_done = s_ready + NB;

  // ---- which (sequence, head, dv block): XCD-aware.  Workgroup b runs on XCD
  // b % 8; the NV dv blocks of one (sequence, head) share an XCD (and its L2),
  // and low ranks (the longest sequences when packed) start first.
  int pidx, vb, lc1 = 0;
  if constexpr (PIPE == 1) {         // (sequence, head, round) of uniform rows
    const int nr = (T + C - 1) / C;
    pidx = (int)(blockIdx.x / (unsigned)nr);
    lc1 = (int)(blockIdx.x % (unsigned)nr);
    vb = 0;
  } else {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    pidx = (slot / NV) * 8 + xcd;
    vb = slot % NV;
  }
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
  // the wave index is uniform: in a scalar register, buffer resources built
  // from it need no per-lane loop
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  if (threadIdx.x < 2 * NB) s_ready[threadIdx.x] = 0;   // ready[], then done[]
  __syncthreads();

  // Global traffic goes through buffer resources based at a block's (or a
  // round's) first token row, with num_records ending at the sequence's last
  // row of this head: rows past the sequence end read as zero and writes to
  // them are dropped, so no lane branches or clamps.
  auto rsrc = [&](const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, kBufferFlags);
  };
  // Slot image of the two-kernel hand-off: the parts of a slot the state pass
  // reads, the row planes and then the (K / gamma')^T units through the mode
  // word, for block b = 4 lc + I of (sequence, head) pidx of uniform rows.
  constexpr int IMG_A = 4 * SL::PL, IMG = IMG_A + (SL::NF - SL::KT);
  auto image = [&](int lcx, int Ix) {
    const size_t nblk = (size_t)((T + CB - 1) / CB);
    return img + ((size_t)pidx * nblk + (size_t)lcx * NB + (size_t)Ix) * IMG;
  };
  auto slot_offset = [](int i) { return i < IMG_A ? SL::GK + i : SL::KT + (i - IMG_A); };

  if (PIPE == 1 || w >= 4) {
    // ======================= preparation: wave 4 + I fills slot I
    const int I = PIPE == 1 ? w : w - 4, sb = I * SLOT;
    if constexpr (PIPE == 2) {
      // the slot images of the preparation kernel, loaded in place of it: a
      // round's image is read into registers while the state pass still works
      // on the slot's previous block, then written once the slot is free
      constexpr int NU = (IMG + 1023) / 1024;      // 16-byte units per lane
      uint4 buf[NU];
      auto fetch = [&](int lc) {
        const char *src = image(lc, I);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int i = 1024 * u + 16 * lane;
          if (i < IMG) buf[u] = *reinterpret_cast<const uint4 *>(src + i);
        }
      };
      if (CB * I < len) fetch(0);
      for (int lc = 0; lc < nch; ++lc) {
        if (lc * C + CB * I >= len) break;
        wait_for(s_done + I, 4 * lc);    // the state pass is done with the slot
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int i = 1024 * u + 16 * lane;
          if (i < IMG) lds_put(smem, sb + slot_offset(i), buf[u]);
        }
        publish(s_ready + I, lc + 1, lane == 0);
        if ((lc + 1) * C + CB * I < len) fetch(lc + 1);
      }
      return;
    }

    const int tg = lane / CG, cg = lane % CG, ca = PG::base(cg);
    float4 in_a[TPL][2];
    uint4 in_k[TPL], in_q[TPL];
    float in_b = 0.f;
    auto load = [&](int lc) {
      const int tb = lc * C + CB * I;
      const int nbt = min(CB, len - tb);
      const size_t row0 = (size_t)(start + tb) * H + h;
      const int rsg = H * DK * 4, rsk = H * DK * 2;
      const auto rg = rsrc(g + row0 * DK, (nbt - 1) * rsg + DK * 4);
      const auto rk = rsrc(k + row0 * DK, (nbt - 1) * rsk + DK * 2);
      const auto rq = rsrc(q + row0 * DK, (nbt - 1) * rsk + DK * 2);
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const int t = tg * TPL + r;
        in_a[r][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, t * rsg + 4 * ca, 0, 0));
        in_a[r][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, t * rsg + 4 * ca + 64, 0, 0));
        const uint2 k0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, t * rsk + 2 * ca, 0, 0));
        const uint2 k1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, t * rsk + 2 * ca + 32, 0, 0));
        const uint2 q0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, t * rsk + 2 * ca, 0, 0));
        const uint2 q1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, t * rsk + 2 * ca + 32, 0, 0));
        in_k[r] = make_uint4(k0.x, k0.y, k1.x, k1.y);
        in_q[r] = make_uint4(q0.x, q0.y, q1.x, q1.y);
      }
      const auto rb = rsrc(beta + row0, (nbt - 1) * H * 4 + 4);
      in_b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
    };
    const int lc_lo = PIPE == 1 ? lc1 : 0, lc_hi = PIPE == 1 ? lc1 + 1 : nch;
    if (lc_lo * C + CB * I < len) load(lc_lo);

    for (int lc = lc_lo; lc < lc_hi; ++lc) {
      const int tb = lc * C + CB * I;
      if (tb >= len) break;              // past the sequence end (last round only)
      const int nbt = min(CB, len - tb);
      if (nbt < CB) {                    // padding tokens: identity gate, zero key and query
#pragma unroll
        for (int r = 0; r < TPL; ++r)
          if (tg * TPL + r >= nbt) {
            in_a[r][0] = make_float4(1.f, 1.f, 1.f, 1.f);
            in_a[r][1] = in_a[r][0];
            in_k[r] = make_uint4(0u, 0u, 0u, 0u);
            in_q[r] = in_k[r];
          }
      }
      // q/k normalisation factors (sum of squares + 1e-6)^(-1/2) of each token:
      // the CG lanes of a token group hold one token's channels.  They go to the
      // slot's table (a region only this wave touches) and are read back where
      // needed, which spares registers.
      if (NORM) {
#pragma unroll
        for (int r = 0; r < TPL; ++r) {
          float sk = 0.f, sq = 0.f;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float kk = bf16_of(in_k[r], cc), qq = bf16_of(in_q[r], cc);
            sk += kk * kk;
            sq += qq * qq;
          }
#pragma unroll
          for (int m = 1; m < CG; m <<= 1) {
            sk += __shfl_xor(sk, m);
            sq += __shfl_xor(sq, m);
          }
          if (cg == 0)
            lds_put(smem, sb + SL::NF + 8 * (tg * TPL + r),
                    make_float2(__builtin_amdgcn_rsqf(sk + 1e-6f), __builtin_amdgcn_rsqf(sq + 1e-6f)));
        }
      }
      auto norm_factors = [&](int r, float &fk, float &fq) {
        fk = 1.f;
        fq = 1.f;
        if (NORM) {
          const float2 f = lds_at<float2>(smem, sb + SL::NF, 8 * (tg * TPL + r));
          fk = f.x;
          fq = f.y;
        }
      };

      // ---- gate products.  Each gate's magnitude is floored at 2^-126 (a NaN
      // gate counts as that floor, with its sign bit); KDA mode takes |alpha|.
      auto gate = [&](int r, int cc) {
        const float4 &v = in_a[r][cc >> 2];
        const float a = (cc & 3) == 0 ? v.x : (cc & 3) == 1 ? v.y : (cc & 3) == 2 ? v.z : v.w;
        const float m = fmaxf(fabsf(a), kGateFloor);
        return SIGNED ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, m) |
                                                      (__builtin_bit_cast(uint32_t, a) & 0x80000000u))
                      : m;
      };
      // lane-local: the product of the lane's gates, and the extremes of the
      // products of the gates after each of its tokens (within the lane)
      auto lane_products = [&](float (&tp)[8], float (&smin)[8], float (&smax)[8]) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) { tp[cc] = 1.f; smin[cc] = 1.f; smax[cc] = 1.f; }
#pragma unroll
        for (int r = TPL - 1; r >= 0; --r)
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            if (r < TPL - 1) {
              smin[cc] = fminf(smin[cc], fabsf(tp[cc]));
              smax[cc] = fmaxf(smax[cc], fabsf(tp[cc]));
            }
            tp[cc] *= gate(r, cc);
          }
      };
      float tp[8], smin[8], smax[8];
      lane_products(tp, smin, smax);
      // across token groups: exS = product of the gates of all later groups,
      // gn = gamma_n, the product of all sixteen
      float exS[8], gn[8];
#pragma unroll
      for (int d = 1; d < TG; d <<= 1)
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const float y = __shfl_down(tp[cc], d * CG);
          if (tg + d < TG) tp[cc] *= y;
        }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const float y = __shfl_down(tp[cc], CG);
        exS[cc] = tg + 1 < TG ? y : 1.f;
        gn[cc] = __shfl(tp[cc], cg);
      }
      // the factored form needs every gamma_n / gamma_t within 2^+-110
      bool bad = false;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const float e = fabsf(exS[cc]);
        bad |= !(e * smax[cc] <= kGuardScale && e * smin[cc] >= 1.f / kGuardScale);
      }
      const bool exact = __any(bad);

      // ---- the slot is free once the state pass is done with the previous round
      if constexpr (PIPE == 0) wait_for(s_done + I, 4 * lc);

      // (K / gamma')^T of tokens t0 = tg * TPL + r2 and t0 + 1 (hi and lo words
      // of eight channels each): per channel, the hi and lo words of the token
      // pair go to their fragment unit in one 8-byte store
      // (K / gamma')^T of tokens t0 = tg * TPL + r2 and t0 + 1: per channel, the
      // hi and lo words of the pair (two tokens each).  A unit holds, for tokens
      // 4g .. 4g+3, [hi 4g,4g+1 | hi 4g+2,4g+3 | lo 4g,4g+1 | lo 4g+2,4g+3], so the
      // state pass reads both 8-byte fragments in place.  Four tokens per lane
      // (dk = 128): the later pair's words wait in ph/pl and each unit is one
      // 16-byte store; two (dk = 64): one 4-byte store per word.
      uint32_t ph[8], pl[8];
      auto kt_store = [&](int r2, const uint32_t (&kwh)[2][4], const uint32_t (&kwl)[2][4]) {
        // channel ca + (cc & 3) + 16 (cc >> 2) sits in tile 2 (cg / 4) + (cc >> 2), row
        // 4 (cg % 4) + (cc & 3): a lane base plus a constant per cc
        const int t0 = tg * TPL + r2;
        const int kb = sb + SL::KT + 16 * kt_unit(2 * (cg >> 2), t0 >> 2, 4 * (cg & 3));
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          // half-word cc & 1 of token t0's word, then of token t0 + 1's, in one byte
          // permute (bytes 0-3 select from the second operand, 4-7 from the first)
          const int wd = cc >> 1;
          const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t hw = __builtin_amdgcn_perm(kwh[1][wd], kwh[0][wd], sel);
          const uint32_t lw = __builtin_amdgcn_perm(kwl[1][wd], kwl[0][wd], sel);
          const int ko = kb + 16 * kt_unit(cc >> 2, 0, cc & 3);
          if (TPL == 4) {
            if (r2 == 2) {
              ph[cc] = hw;
              pl[cc] = lw;
            } else {
              lds_put(smem, ko, make_uint4(hw, ph[cc], lw, pl[cc]));
            }
          } else {
            const int pw = 4 * ((t0 >> 1) & 1);
            lds_put(smem, ko + pw, hw);
            lds_put(smem, ko + 8 + pw, lw);
          }
        }
      };

      // ---- A and P tiles from the KG, GK and GQ planes in the slot, computed
      // transposed: the MFMA's row operand is the column plane (K/gamma' in the
      // factored form), its column operand -(gamma' K) or gamma' Q, so lane (g, l)
      // holds row l and columns 4g .. 4g+3.  The wave reads only what it wrote,
      // and LDS serves one wave's accesses in order.
      auto ap_tiles = [&](f32x4 &pA, f32x4 &pP, int col_plane) {
        const int l = lane & 15, gg = lane >> 4;
        const int rb = sb + 2 * (l * SL::RW + 8 * gg);
        pA = f32x4{0.f, 0.f, 0.f, 0.f};
        pP = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 ka_h = frag32p(smem, rb + col_plane, 64 * kb);
          const bf16x8 ka_l = frag32p(smem, rb + col_plane + SL::PL, 64 * kb);
          const bf16x8 rk_h = frag32p(smem, rb + SL::GK, 64 * kb);
          const bf16x8 rk_l = frag32p(smem, rb + SL::GK + SL::PL, 64 * kb);
          const bf16x8 rq_h = frag32p(smem, rb + SL::GQ, 64 * kb);
          const bf16x8 rq_l = frag32p(smem, rb + SL::GQ + SL::PL, 64 * kb);
          pA = mfma32(ka_l, rk_h, pA);     // A and P alternate (independent chains)
          pP = mfma32(ka_l, rq_h, pP);
          pA = mfma32(ka_h, rk_l, pA);
          pP = mfma32(ka_h, rq_l, pP);
          pA = mfma32(ka_h, rk_h, pA);
          pP = mfma32(ka_h, rq_h, pP);
        }
      };
      // pA holds -A_lj / beta_l: row l of A, zero on and above the diagonal, to
      // the fp32 store; row l of P to its fragment unit (l, g).  `bcur` holds
      // beta of token `lane`.
      auto ap_store = [&](const f32x4 &pA, const f32x4 &pP, float bcur) {
        const int l = lane & 15, gg = lane >> 4;
        const float bl = __shfl(bcur, l);
        float av[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * gg + e;
          av[e] = j < l ? -pA[e] * bl : 0.f;
          pv[e] = j <= l ? pP[e] : 0.f;
        }
        lds_put(smem, sb + SL::AD + 4 * (l * ADS + 4 * gg), make_float4(av[0], av[1], av[2], av[3]));
        uint2 hh, ll;
        split_quad(pv, hh, ll);
        lds_put(smem, sb + SL::PT + 16 * lane, make_uint4(hh.x, hh.y, ll.x, ll.y));
      };
      // the lane's eight channels of token t, split hi/lo, as one 16-byte run of
      // a permuted [CB][DK] row plane
      auto put_row = [&](int region, int t, const float (&x)[8]) {
        const int ro = 2 * (t * SL::RW + 8 * cg);
        uint2 h0, l0, h1, l1;
        split_quad(*reinterpret_cast<const float(*)[4]>(x), h0, l0);
        split_quad(*reinterpret_cast<const float(*)[4]>(x + 4), h1, l1);
        lds_put(smem, sb + region + ro, make_uint4(h0.x, h0.y, h1.x, h1.y));
        lds_put(smem, sb + region + SL::PL + ro, make_uint4(l0.x, l0.y, l1.x, l1.y));
      };

      // The keys and queries as values the compiler must reload: a pass that
      // recomputes its operands from them does not keep another pass's alive.
      auto opaque_inputs = [&]() {
#pragma unroll
        for (int r = 0; r < TPL; ++r) {
          asm volatile("" : "+v"(in_k[r].x), "+v"(in_k[r].y), "+v"(in_k[r].z), "+v"(in_k[r].w));
          asm volatile("" : "+v"(in_q[r].x), "+v"(in_q[r].y), "+v"(in_q[r].z), "+v"(in_q[r].w));
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            asm volatile("" : "+v"(in_a[r][hf].x), "+v"(in_a[r][hf].y), "+v"(in_a[r][hf].z),
                         "+v"(in_a[r][hf].w));
        }
      };

      // ---- exact blocks.  G (the cumulative sum of log2|alpha| from the block
      // start, each term floored at -126) and the cumulative parity of negative
      // gates, per (token, channel), in registers.
      // the lane's token r, channels 4 hf .. 4 hf + 3, of the slot's fp32 [CB][DK]
      // table (G, then the state pass's row factors)
      auto g_at = [&](int r, int hf) {
        return lds_at<float4>(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca), 64 * hf);
      };

      // ---- operands: rows gamma' K and gamma' Q, columns K / gamma'.  Factored:
      // gamma' = gamma_t / gamma_n = 1 / (product of the gates after t), a running
      // product going backwards from the block end.  Exact: rows gamma_t (from the
      // block start) and columns gamma_n / gamma_t, from G.  One copy of the loop
      // per block kind, so neither carries the other's values.
      auto operand_planes = [&](auto kind) {
      constexpr bool EX = decltype(kind)::value;
      float run[8];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) run[cc] = exS[cc];
#pragma unroll
      for (int r2 = TPL - 2; r2 >= 0; r2 -= 2) {
        uint32_t kwh[2][4], kwl[2][4];
#pragma unroll
        for (int u = 1; u >= 0; --u) {
          const int r = r2 + u, t = tg * TPL + r;
          float fk, fq;
          norm_factors(r, fk, fq);
          float gam8[8], kf8[8];
          if constexpr (!EX) {
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              const float sa = run[cc];                      // gamma_n / gamma_t
              gam8[cc] = __builtin_amdgcn_rcpf(sa);         // gamma'
              kf8[cc] = sa;
              run[cc] = sa * gate(r, cc);
            }
          } else {
            const float4 g0 = g_at(r, 0), g1 = g_at(r, 1);  // gamma_t from the block start
            const float G8[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              gam8[cc] = G8[cc];
              kf8[cc] = run[cc];                             // gamma_n / gamma_t
              run[cc] *= gate(r, cc);
            }
          }
          float gk[8], gq[8], kg[8];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float kk = bf16_of(in_k[r], cc) * fk, qq = bf16_of(in_q[r], cc) * fq;
            gk[cc] = -kk * gam8[cc];
            gq[cc] = qq * gam8[cc];
            kg[cc] = kk * kf8[cc];
          }
          // the lane's eight channels are one 16-byte run of the permuted row
          const int ro = 2 * (t * SL::RW + 8 * cg);
          uint2 h0, l0, h1, l1;
          split_quad(*reinterpret_cast<const float(*)[4]>(gk), h0, l0);
          split_quad(*reinterpret_cast<const float(*)[4]>(gk + 4), h1, l1);
          lds_put(smem, sb + SL::GK + ro, make_uint4(h0.x, h0.y, h1.x, h1.y));
          lds_put(smem, sb + SL::GK + SL::PL + ro, make_uint4(l0.x, l0.y, l1.x, l1.y));
          split_quad(*reinterpret_cast<const float(*)[4]>(gq), h0, l0);
          split_quad(*reinterpret_cast<const float(*)[4]>(gq + 4), h1, l1);
          lds_put(smem, sb + SL::GQ + ro, make_uint4(h0.x, h0.y, h1.x, h1.y));
          lds_put(smem, sb + SL::GQ + SL::PL + ro, make_uint4(l0.x, l0.y, l1.x, l1.y));
          split_quad(*reinterpret_cast<const float(*)[4]>(kg), h0, l0);
          split_quad(*reinterpret_cast<const float(*)[4]>(kg + 4), h1, l1);
          if constexpr (!EX) {   // the exact path keeps its G table in this region
            lds_put(smem, sb + SL::KG + ro, make_uint4(h0.x, h0.y, h1.x, h1.y));
            lds_put(smem, sb + SL::KG + SL::PL + ro, make_uint4(l0.x, l0.y, l1.x, l1.y));
          }
          kwh[u][0] = h0.x; kwh[u][1] = h0.y; kwh[u][2] = h1.x; kwh[u][3] = h1.y;
          kwl[u][0] = l0.x; kwl[u][1] = l0.y; kwl[u][2] = l1.x; kwl[u][3] = l1.y;
        }
        kt_store(r2, kwh, kwl);
        __builtin_amdgcn_sched_barrier(0);   // two tokens at a time: bounded live range
      }
      };

      if (exact) {
        // Half-block references: every ratio gamma_i / gamma_j (j <= i) splits as
        // (gamma_i / gamma_ref)(gamma_ref / gamma_j) about the last token of j's
        // half (token 7 or 15).  Inside a half that is the factored form of an
        // eight-token block; for i in the second half and j in the first, both
        // factors are products of gates (no inverse), so a decaying gate can only
        // make them small.  The tiles are two matrix-core passes: rows and columns
        // referenced to their own half's end, then the second half's rows
        // referenced to token 7 against the same columns.  Every factor is a
        // running product of the signed gates.
        //   eh: product of the later token groups of the lane's half,
        //   ph: product of the earlier token groups of the lane's half,
        //   pp: product of all earlier token groups (from the block start).
        constexpr int GH = TG / 2;                 // token groups per half
        const int th = tg % GH;                    // the lane's group within its half
        const bool second = tg >= GH;              // the lane's tokens are in the second half
        opaque_inputs();
        float eh[8], ph[8];
        bool wide = false;
        {
          float tl[8], mn[8], mx[8], sh[8];
          lane_products(tl, mn, mx);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) { sh[cc] = tl[cc]; ph[cc] = tl[cc]; }
#pragma unroll
          for (int d = 1; d < GH; d <<= 1)
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              const float y = __shfl_down(sh[cc], d * CG), z = __shfl_up(ph[cc], d * CG);
              if (th + d < GH) sh[cc] *= y;
              if (th >= d) ph[cc] *= z;
            }
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float y = __shfl_down(sh[cc], CG), z = __shfl_up(ph[cc], CG);
            eh[cc] = th + 1 < GH ? y : 1.f;
            ph[cc] = th ? z : 1.f;
            // the half's factors within 2^+-110
            const float e = fabsf(eh[cc]);
            wide |= !(e * mx[cc] <= kGuardScale && e * mn[cc] >= 1.f / kGuardScale);
          }
        }
        // the state pass's row factors gamma_t (from the block start) to the
        // slot's table: pp, the product of all earlier token groups, times the
        // lane's running product
        auto gamma_table = [&]() {
          float tl[8], mn[8], mx[8], pr[8];
          lane_products(tl, mn, mx);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) pr[cc] = tl[cc];
#pragma unroll
          for (int d = 1; d < TG; d <<= 1)
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              const float y = __shfl_up(pr[cc], d * CG);
              if (tg >= d) pr[cc] *= y;
            }
          float run[8];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float x = __shfl_up(pr[cc], CG);
            run[cc] = tg ? x : 1.f;
          }
#pragma unroll
          for (int r = 0; r < TPL; ++r) {
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) run[cc] *= gate(r, cc);
            lds_put(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca),
                    make_float4(run[0], run[1], run[2], run[3]));
            lds_put(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca) + 64,
                    make_float4(run[4], run[5], run[6], run[7]));
          }
        };
        if (!__any(wide)) {
          gamma_table();
          // pass one: columns kappa_t = gamma_ref / gamma_t (the product of the
          // half's gates after t), rows 1 / kappa_t
          float run[8];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) run[cc] = eh[cc];
#pragma unroll
          for (int r = TPL - 1; r >= 0; --r) {
            float fk, fq;
            norm_factors(r, fk, fq);
            float gk[8], gq[8], kg[8];
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              const float kap = run[cc], rho = __builtin_amdgcn_rcpf(kap);
              run[cc] = kap * gate(r, cc);
              const float kk = bf16_of(in_k[r], cc) * fk, qq = bf16_of(in_q[r], cc) * fq;
              gk[cc] = -kk * rho;
              gq[cc] = qq * rho;
              kg[cc] = kk * kap;
            }
            const int t = tg * TPL + r;
            put_row(SL::GK, t, gk);
            put_row(SL::GQ, t, gq);
            put_row(SL::KT, t, kg);
            __builtin_amdgcn_sched_barrier(0);   // a token at a time: bounded live range
          }
          f32x4 pA1, pP1, pA2, pP2;
          ap_tiles(pA1, pP1, SL::KT);
          opaque_inputs();
          // pass two: the second half's rows gamma_t / gamma_7 (the product of the
          // gates from token 8 to t); the first half's rows keep pass one's values,
          // whose results are not used
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) run[cc] = ph[cc];
#pragma unroll
          for (int r = 0; r < TPL; ++r) {
            float fk, fq;
            norm_factors(r, fk, fq);
            float gk[8], gq[8];
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              run[cc] *= gate(r, cc);
              const float kk = bf16_of(in_k[r], cc) * fk, qq = bf16_of(in_q[r], cc) * fq;
              gk[cc] = -kk * run[cc];
              gq[cc] = qq * run[cc];
            }
            if (second) {
              const int t = tg * TPL + r;
              put_row(SL::GK, t, gk);
              put_row(SL::GQ, t, gq);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          ap_tiles(pA2, pP2, SL::KT);
          opaque_inputs();
          // row l in the second half and columns 4g .. 4g+3 in the first: pass two
          const bool cross = (lane & 15) >= CB / 2 && 4 * (lane >> 4) < CB / 2;
          ap_store(cross ? pA2 : pA1, cross ? pP2 : pP1, in_b);
        } else {
          // A fall beyond 2^-110 inside a half: A and P element by element from
          // fp32 ratios 2^(G_i - G_j), with G (the cumulative sum of log2|alpha|,
          // each term floored at -126) and the cumulative parities of negative
          // gates in tables in the slot.
          float tot[8];
          uint32_t ptot = 0u, pbits = 0u;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) tot[cc] = 0.f;
#pragma unroll
          for (int r = 0; r < TPL; ++r) {
            const float a8[8] = {in_a[r][0].x, in_a[r][0].y, in_a[r][0].z, in_a[r][0].w,
                                 in_a[r][1].x, in_a[r][1].y, in_a[r][1].z, in_a[r][1].w};
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              tot[cc] += fmaxf(flog2(fabsf(a8[cc])), kLog2Floor);
              if (SIGNED) ptot ^= (__builtin_bit_cast(uint32_t, a8[cc]) >> 31) << cc;
            }
            lds_put(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca),
                    make_float4(tot[0], tot[1], tot[2], tot[3]));
            lds_put(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca) + 64,
                    make_float4(tot[4], tot[5], tot[6], tot[7]));
            pbits |= ptot << (8 * r);
          }
          // the earlier token groups' sums (and parities) are added to the lane's
#pragma unroll
          for (int d = 1; d < TG; d <<= 1) {
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
              const float y = __shfl_up(tot[cc], d * CG);
              if (tg >= d) tot[cc] += y;
            }
            if (SIGNED) {
              const uint32_t y = __shfl_up(ptot, d * CG);
              if (tg >= d) ptot ^= y;
            }
          }
          float ex[8];
          uint32_t exP = 0u;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float y = __shfl_up(tot[cc], CG);
            ex[cc] = tg ? y : 0.f;
          }
          if (SIGNED) {
            const uint32_t y = __shfl_up(ptot, CG);
            exP = tg ? y : 0u;
          }
#pragma unroll
          for (int r = 0; r < TPL; ++r)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              float4 gg = g_at(r, hf);
              gg.x += ex[4 * hf]; gg.y += ex[4 * hf + 1]; gg.z += ex[4 * hf + 2]; gg.w += ex[4 * hf + 3];
              lds_put(smem, sb + SL::XG + 4 * ((tg * TPL + r) * DK + ca) + 64 * hf, gg);
            }
          {
            uint32_t pw = 0u;
#pragma unroll
            for (int r = 0; r < TPL; ++r) pw |= ((exP ^ (pbits >> (8 * r))) & 0xFFu) << (8 * r);
            lds_put(smem, sb + SL::XP + 4 * lane, pw);
          }
          const size_t row0 = (size_t)(start + tb) * H + h;
          const int rsk = H * DK * 2;
          exact_tiles<DK, SIGNED, NORM>(smem, sb, lane, __shfl(in_b, lane >> 2),
                                        rsrc(k + row0 * DK, (nbt - 1) * rsk + DK * 2),
                                        rsrc(q + row0 * DK, (nbt - 1) * rsk + DK * 2), rsk);
          gamma_table();   // over the G table, which the tiles have finished reading
        }
        operand_planes(Kind<true>{});
      } else {
        operand_planes(Kind<false>{});
      }

      // The block's inputs are consumed (beta aside): the next round's block is
      // loaded now, in flight during the tiles and the inverse.
      const float cur_b = in_b;
      if (PIPE == 0 && (lc + 1) * C + CB * I < len) load(lc + 1);

      if (!exact) {
        f32x4 pA, pP;
        ap_tiles(pA, pP, SL::KG);
        ap_store(pA, pP, cur_b);
      }

      // ---- state factor gamma_n, beta, mode
      if (tg == 0) {
        lds_put(smem, sb + SL::PRE + 4 * ca, make_float4(gn[0], gn[1], gn[2], gn[3]));
        lds_put(smem, sb + SL::PRE + 4 * ca + 64, make_float4(gn[4], gn[5], gn[6], gn[7]));
      }
      if (lane < CB) lds_put(smem, sb + SL::BT + 4 * lane, cur_b);
      if (lane == 0) lds_put(smem, sb + SL::MODE, exact ? 1 : 0);
      // ---- T = (I + A)^-1, row i per quad of lanes: lane 4i + q holds T[i][4q ..
      // 4q+3].  T (I + A) = I gives T[i][j] = delta_ij - sum_{k > j} T[i][k] A[k][j];
      // for k from 15 down, T[i][k] is then final: it is broadcast within the
      // quad and, times row k of A (zero from column k on), subtracted from the
      // quad's columns.  The finished row goes to fragment unit (i, q).
      {
        const int i = lane >> 2, q = lane & 3;
        const int adq = sb + SL::AD + 16 * q;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == i) ? 1.f : 0.f;
        float4 ar[2];
        ar[(CB - 1) & 1] = lds_at<float4>(smem, adq, 4 * (CB - 1) * ADS);
#pragma unroll
        for (int kk = CB - 1; kk >= 1; --kk) {
          if (kk > 1) ar[(kk - 1) & 1] = lds_at<float4>(smem, adq, 4 * (kk - 1) * ADS);
          const float tk = quad_bcast(x[kk & 3], kk >> 2);
          const float4 &a = ar[kk & 1];
          x[0] -= tk * a.x;
          x[1] -= tk * a.y;
          x[2] -= tk * a.z;
          x[3] -= tk * a.w;
        }
        uint2 hh, ll;
        split_quad(x, hh, ll);
        lds_put(smem, sb + SL::TT + 16 * (16 * q + i), make_uint4(hh.x, hh.y, ll.x, ll.y));
      }

      // ---- hand the slot over (two-kernel hand-off: write its image)
      if constexpr (PIPE == 1) {
        char *dst = image(lc, I);
        for (int i = 16 * lane; i < IMG; i += 16 * 64)
          *reinterpret_cast<uint4 *>(dst + i) = lds_at<uint4>(smem, sb + slot_offset(i), 0);
      } else {
        publish(s_ready + I, lc + 1, lane == 0);
      }
    }
  } else if constexpr (PIPE != 1) {
    // ======================= state pass (waves 0-3)
    const int l16 = lane & 15, gq = lane >> 4;
    const int col = vb * BV + 16 * w + l16;
    f32x4 accS[ST];
#pragma unroll
    for (int tt = 0; tt < ST; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accS[tt][e] = S0 ? S0[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] : 0.f;
    // the initial state is in registers before the loop, so no wait inside the
    // loop is charged with these loads (vmcnt(0); expcnt, lgkmcnt untouched)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const int lpD = 2 * (l16 * SL::RW + 8 * gq);
    const int rs_v = H * DV * 2;
    // v, two blocks ahead: block b of a round reads ring entry b, so every
    // index is known at compile time and the wait for a load falls at its use
    unsigned short nv[NB][4];
    auto load_v = [&](int lc, int I) {
      const int t0 = start + lc * C, nt = min(C, len - lc * C);
      const auto rv = rsrc(v + ((size_t)t0 * H + h) * DV, (nt - 1) * rs_v + DV * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        nv[I][e] = __builtin_amdgcn_raw_buffer_load_b16(rv, (CB * I + 4 * gq + e) * rs_v + 2 * col, 0, 0);
    };
    static_assert(NB >= 3, "the v ring holds the current block and the next two");
    if (nch > 0) {      // rows past the sequence end read as zero
      load_v(0, 0);
      load_v(0, 1);
    }

    for (int lc = 0; lc < nch; ++lc) {
      const int t0 = start + lc * C, nt = min(C, len - lc * C);
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        if (CB * I >= nt) break;
        if (I + 2 < NB) {
          if (CB * (I + 2) < nt) load_v(lc, I + 2);
        } else if (lc + 1 < nch) {
          load_v(lc + 1, I + 2 - NB);
        }
        const unsigned short(&cv)[4] = nv[I];

        wait_for(s_ready + I, lc + 1);
        const int sb = I * SLOT;
        // Reads in the order they are needed, all issued before the first wait:
        // the mode, gamma_n, the first k block's operand fragments, then T, P
        // and beta (needed after the X and O products).
        const int mode = lds_at<int>(smem, sb, SL::MODE);
        __builtin_amdgcn_sched_barrier(0);
        float4 gnv[ST];
#pragma unroll
        for (int tt = 0; tt < ST; ++tt)
          gnv[tt] = lds_at<float4>(smem, sb + SL::PRE, 4 * (16 * tt + 4 * gq));
        __builtin_amdgcn_sched_barrier(0);
        const int gkb = sb + SL::GK + lpD, gqb = sb + SL::GQ + lpD;
        bf16x8 fk_h[2], fk_l[2], fq_h[2], fq_l[2];
        auto ld = [&](int kb) {
          const int s = kb & 1;
          fk_h[s] = frag32p(smem, gkb, 64 * kb);
          fk_l[s] = frag32p(smem, gkb, SL::PL + 64 * kb);
          fq_h[s] = frag32p(smem, gqb, 64 * kb);
          fq_l[s] = frag32p(smem, gqb, SL::PL + 64 * kb);
        };
        ld(0);
        const uint4 tw = lds_at<uint4>(smem, sb + SL::TT + 16 * lane, 0);
        const uint4 pw = lds_at<uint4>(smem, sb + SL::PT + 16 * lane, 0);
        const float4 bq = lds_at<float4>(smem, sb + SL::BT, 16 * gq);
        __builtin_amdgcn_sched_barrier(0);
        const int exact = __builtin_amdgcn_readfirstlane(mode);
        // ---- S_pre = Diag(gamma_n) S (factored blocks), split for the products
        if (!exact) {
#pragma unroll
          for (int tt = 0; tt < ST; ++tt) {
            const float4 gn = gnv[tt];
            accS[tt][0] *= gn.x; accS[tt][1] *= gn.y; accS[tt][2] *= gn.z; accS[tt][3] *= gn.w;
          }
        }
        bf16x8 sh[KB], sl[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) split8_acc(accS[2 * kb], accS[2 * kb + 1], sh[kb], sl[kb]);
        // ---- X = V - (gamma' K) S_pre;  O = (gamma' Q) S_pre
        f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accO = {0.f, 0.f, 0.f, 0.f};
        uint4 kw[ST];     // (K/gamma')^T fragment units, read once the operand reads are out
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (kb + 1 < KB) {
            ld(kb + 1);
          } else {
#pragma unroll
            for (int tt = 0; tt < ST; ++tt)
              kw[tt] = lds_at<uint4>(smem, sb + SL::KT + 16 * kt_unit(0, gq, l16), 16 * kt_unit(tt, 0, 0));
          }
          __builtin_amdgcn_sched_barrier(0);
          const int s = kb & 1;
          // X and O alternate, so each product waits on its chain two
          // instructions back rather than one
          accX = mfma32(fk_l[s], sh[kb], accX);
          accO = mfma32(fq_l[s], sh[kb], accO);
          accX = mfma32(fk_h[s], sl[kb], accX);
          accO = mfma32(fq_h[s], sl[kb], accO);
          accX = mfma32(fk_h[s], sh[kb], accX);
          accO = mfma32(fq_h[s], sh[kb], accO);
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- U = (I + A)^-1 Diag(beta) X
        f32x4 y;
        y[0] = bq.x * (accX[0] + bf16_to_f32(cv[0]));
        y[1] = bq.y * (accX[1] + bf16_to_f32(cv[1]));
        y[2] = bq.z * (accX[2] + bf16_to_f32(cv[2]));
        y[3] = bq.w * (accX[3] + bf16_to_f32(cv[3]));
        // each three-term product is two 16x16x32 MFMAs of the fragment unit
        // [hi | lo]: against [b_hi | b_hi], then against [b_lo | 0]
        const bf16x4 z4 = {};
        bf16x4 yh, yl;
        split4(y, yh, yl);
        f32x4 u = {0.f, 0.f, 0.f, 0.f}, u2 = {0.f, 0.f, 0.f, 0.f};
        u = mfma32(as_frag8(tw), cat8(yh, yh), u);
        u2 = mfma32(as_frag8(tw), cat8(yl, z4), u2);
        u += u2;
        bf16x4 uh, ul;
        split4(u, uh, ul);
        const bf16x8 uu = cat8(uh, uh), ul0 = cat8(ul, z4);
        // ---- O += P U;  S <- S_pre + (K/gamma')^T U  (exact: Diag(gamma_n) S + ...)
        accO = mfma32(as_frag8(pw), uu, accO);
        if (exact) {
#pragma unroll
          for (int tt = 0; tt < ST; ++tt) {
            const float4 gn = lds_at<float4>(smem, sb + SL::PRE, 4 * (16 * tt + 4 * gq));
            accS[tt][0] *= gn.x; accS[tt][1] *= gn.y; accS[tt][2] *= gn.z; accS[tt][3] *= gn.w;
          }
        }
        // all hi terms, then all lo terms: no product waits on the one before
#pragma unroll
        for (int tt = 0; tt < ST; ++tt) accS[tt] = mfma32(as_frag8(kw[tt]), uu, accS[tt]);
        accO = mfma32(as_frag8(pw), ul0, accO);
#pragma unroll
        for (int tt = 0; tt < ST; ++tt) accS[tt] = mfma32(as_frag8(kw[tt]), ul0, accS[tt]);
        count_done(s_done + I, lane == 0);
        // ---- store o (rows past the sequence end are dropped by the resource)
        if (OBF16) {
          const int rs = H * DV * 2;
          const auto ro = rsrc(static_cast<__hip_bfloat16 *>(o) + ((size_t)t0 * H + h) * DV,
                               (nt - 1) * rs + DV * 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const __bf16 bv = (__bf16)accO[e];
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, bv), ro,
                                                  (CB * I + 4 * gq + e) * rs + 2 * col, 0, 0);
          }
        } else {
          const int rs = H * DV * 4;
          const auto ro = rsrc(static_cast<float *>(o) + ((size_t)t0 * H + h) * DV,
                               (nt - 1) * rs + DV * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // through a scalar: a bit_cast of the vector element itself reads element 0
            const float val = accO[e];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), ro,
                                                  (CB * I + 4 * gq + e) * rs + 4 * col, 0, 0);
          }
        }
      }
    }
    if (S_T) {
#pragma unroll
      for (int tt = 0; tt < ST; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S_T[(((size_t)n * H + h) * DK + 16 * tt + 4 * gq + e) * DV + col] = accS[tt][e];
    }
  }
}

template <int DK, bool SIGNED, bool NORM, bool OBF16, int PIPE = 0>
hipError_t launch_dk(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                     int DV, int N, SeqTable tab, int packed, hipStream_t stream,
                     char *img = nullptr) {
  const int NH = N * H, NV = DV / BV;
  const int groups = (NH + 7) / 8;
  dim3 grid((unsigned)groups * 8u * (unsigned)NV), block(NT);
  if (PIPE == 1) {
    grid = dim3((unsigned)NH * (unsigned)((T + C - 1) / C));
    block = dim3(NT / 2);          // the four preparation waves
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<DK, SIGNED, NORM, OBF16, PIPE>), grid, block, 0, stream,
                     static_cast<const __hip_bfloat16 *>(q), static_cast<const __hip_bfloat16 *>(k),
                     static_cast<const __hip_bfloat16 *>(v), g, beta, S0, o, S_T, T, H, DV, NH, NV,
                     tab, packed, img);
  return hipGetLastError();
}

// The two-kernel hand-off: the preparation kernel, then the state kernel.
template <int DK, bool SIGNED>
hipError_t launch_split(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *S0, void *o, float *S_T, int T, int H,
                        int DV, int N, SeqTable tab, char *img, hipStream_t stream) {
  if (T == 0) return launch_dk<DK, SIGNED, false, false, 0>(q, k, v, g, beta, S0, o, S_T, T, H,
                                                             DV, N, tab, 0, stream);
  hipError_t e = launch_dk<DK, SIGNED, false, false, 1>(q, k, v, g, beta, S0, o, S_T, T, H, DV, N,
                                                        tab, 0, stream, img);
  if (e != hipSuccess) return e;
  return launch_dk<DK, SIGNED, false, false, 2>(q, k, v, g, beta, S0, o, S_T, T, H, DV, N, tab,
                                                0, stream, img);
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

size_t fwd_bf16_split_bytes(int T, int H, int dk, int N) {
  const size_t blocks = (size_t)N * H * (size_t)((T + CB - 1) / CB);
  auto image = [](auto slot) {
    using SL = decltype(slot);
    return (size_t)(4 * SL::PL + (SL::NF - SL::KT));
  };
  return blocks * (dk == 64 ? image(Slot<64>{}) : image(Slot<128>{}));
}

hipError_t launch_fwd_bf16_split(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *S0, void *o, float *S_T, int T,
                                 int H, int dk, int dv, int N, SeqTable tab, int signed_gates,
                                 void *img, hipStream_t stream) {
  char *im = static_cast<char *>(img);
  if (dk == 64)
    return signed_gates
               ? launch_split<64, true>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, im, stream)
               : launch_split<64, false>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, im, stream);
  if (dk == 128)
    return signed_gates
               ? launch_split<128, true>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, im, stream)
               : launch_split<128, false>(q, k, v, g, beta, S0, o, S_T, T, H, dv, N, tab, im, stream);
  return hipErrorInvalidValue;
}

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
