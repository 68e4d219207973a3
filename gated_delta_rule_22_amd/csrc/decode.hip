// Recurrent decode step: one token for N*H independent fp32 states, in place.
//
// Per state (one workgroup):
//   u = S^T (alpha * k),  w = S^T (alpha * q)      column reductions over dk
//   delta = beta (v - u)
//   S <- Diag(alpha) S + k delta^T                  = (I - beta k k^T) Diag(alpha) S + beta k v^T
//   o = w + (k . q) delta                            = S_new^T q
// (update rule: blog post "One update, one quarter turn", ELI5 "The mirror").
//
// The state is read once and written once, so the kernel is bound by HBM
// traffic: 2 * dk * dv * 4 bytes per state and step, plus the small inputs.
// Each thread keeps ROWS x 4 state entries in registers (a float4 column
// strip of ROWS rows), so all loads of a workgroup are issued before the first
// reduction and the state never round-trips through LDS.
#include "ckda_internal.h"

namespace ckda {
namespace {

constexpr int kThreads = 256;
typedef float nf4 __attribute__((ext_vector_type(4)));   // for the non-temporal builtins

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ S,
    float *__restrict__ o) {
  constexpr int kColThreads = DV / 4;               // threads across one row (float4 each)
  constexpr int kRowGroups = kThreads / kColThreads;  // row groups
  constexpr int kRows = DK / kRowGroups;             // rows per thread
  static_assert(kRows * kRowGroups == DK, "dk must split evenly over row groups");

  __shared__ float s_ak[DK], s_aq[DK], s_k[DK], s_a[DK];
  __shared__ float s_kq[kThreads / 64];
  __shared__ float4 s_red_u[kRowGroups][kColThreads];
  __shared__ float4 s_red_w[kRowGroups][kColThreads];

  const int head = blockIdx.x;                       // flat (n, h)
  const int t = threadIdx.x;
  const int cg = t % kColThreads;                    // float4 column
  const int rg = t / kColThreads;                    // row group
  float *Sh = S + (size_t)head * DK * DV;

  // Issue the state loads first: they are the traffic that matters.  They are
  // non-temporal: each state is read once per step and the states of one step
  // exceed the last-level cache, so keeping them cached only evicts other data
  // (measured: about 3% faster per step; non-temporal stores were slower).
  float4 st[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const nf4 x = __builtin_nontemporal_load(
        reinterpret_cast<const nf4 *>(Sh + (size_t)(rg * kRows + r) * DV + cg * 4));
    st[r] = make_float4(x.x, x.y, x.z, x.w);
  }

  float kq = 0.f;
  if (t < DK) {
    const float kk = to_f32(k[(size_t)head * DK + t]);
    const float qq = to_f32(q[(size_t)head * DK + t]);
    const float a = g[(size_t)head * DK + t];
    s_k[t] = kk;
    s_a[t] = a;
    s_ak[t] = a * kk;
    s_aq[t] = a * qq;
    kq = kk * qq;
  }
  // k . q: wave reduction, then across the (at most 2) waves holding channels.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
  if ((t & 63) == 0) s_kq[t >> 6] = kq;
  __syncthreads();

  float4 pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int row = rg * kRows + r;
    const float ak = s_ak[row], aq = s_aq[row];
    pu.x += ak * st[r].x; pu.y += ak * st[r].y; pu.z += ak * st[r].z; pu.w += ak * st[r].w;
    pw.x += aq * st[r].x; pw.y += aq * st[r].y; pw.z += aq * st[r].z; pw.w += aq * st[r].w;
  }
  s_red_u[rg][cg] = pu;
  s_red_w[rg][cg] = pw;
  __syncthreads();

  float4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kRowGroups; ++i) {
    const float4 a = s_red_u[i][cg], b = s_red_w[i][cg];
    u.x += a.x; u.y += a.y; u.z += a.z; u.w += a.w;
    w.x += b.x; w.y += b.y; w.z += b.z; w.w += b.w;
  }
  float kqs = 0.f;
#pragma unroll
  for (int i = 0; i < (DK + 63) / 64; ++i) kqs += s_kq[i];

  const float b = beta[head];
  const TIn *vh = v + (size_t)head * DV + cg * 4;
  float4 d;
  d.x = b * (to_f32(vh[0]) - u.x);
  d.y = b * (to_f32(vh[1]) - u.y);
  d.z = b * (to_f32(vh[2]) - u.z);
  d.w = b * (to_f32(vh[3]) - u.w);

  if (rg == 0) {
    float4 out = {w.x + kqs * d.x, w.y + kqs * d.y, w.z + kqs * d.z, w.w + kqs * d.w};
    *reinterpret_cast<float4 *>(o + (size_t)head * DV + cg * 4) = out;
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int row = rg * kRows + r;
    const float a = s_a[row], kk = s_k[row];
    float4 n;
    n.x = a * st[r].x + kk * d.x;
    n.y = a * st[r].y + kk * d.y;
    n.z = a * st[r].z + kk * d.z;
    n.w = a * st[r].w + kk * d.w;
    *reinterpret_cast<float4 *>(Sh + (size_t)row * DV + cg * 4) = n;
  }
}

template <typename TIn>
hipError_t launch_typed(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, float *S, float *o, int NH, int dk, int dv,
                        hipStream_t stream) {
  const TIn *qq = static_cast<const TIn *>(q);
  const TIn *kk = static_cast<const TIn *>(k);
  const TIn *vv = static_cast<const TIn *>(v);
  dim3 grid(NH), block(kThreads);
#define CKDA_DECODE_CASE(DK_, DV_)                                                        \
  if (dk == DK_ && dv == DV_) {                                                           \
    hipLaunchKernelGGL((decode_kernel<TIn, DK_, DV_>), grid, block, 0, stream, qq, kk, vv, \
                       g, beta, S, o);                                                    \
    return hipGetLastError();                                                             \
  }
  CKDA_DECODE_CASE(64, 64)
  CKDA_DECODE_CASE(64, 128)
  CKDA_DECODE_CASE(128, 64)
  CKDA_DECODE_CASE(128, 128)
#undef CKDA_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *S, float *o, int N, int H, int dk, int dv,
                         int in_dtype, hipStream_t stream) {
  const int NH = N * H;
  if (in_dtype == CKDA_BF16)
    return launch_typed<__hip_bfloat16>(q, k, v, g, beta, S, o, NH, dk, dv, stream);
  return launch_typed<float>(q, k, v, g, beta, S, o, NH, dk, dv, stream);
}

}  // namespace ckda
