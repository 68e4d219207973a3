// C-ABI entry points: argument validation, workspace layout, dispatch.
// Every check runs on the host before anything is enqueued, and touches no
// HIP API, so an invalid call has no side effect.
//
// Debug mode (environment variable CKDA_DEBUG set to anything but "" or "0",
// read at every call): cu_seqlens is copied to the host and checked
// (0 = cu[0] <= ... <= cu[N] = T, else CKDA_ERR_SHAPE), which synchronises
// the stream; and the workspace is filled with NaN before the kernels run, so
// a read of anything they did not write shows up in the outputs.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "ckda_internal.h"

namespace ckda {

size_t f64_record_bytes(int dk, int dv);   // fwd_f64.hip

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FwdLayout fwd_layout(int B, int T, int H, int dk, int dv, int N, int in_dtype) {
  FwdLayout L{};
  L.table_bytes = align256(sizeof(int32_t) * (3 * (size_t)N + 1 + (size_t)N));
  // chunks over all sequences: uniform rows give B * ceil(T / C); packed
  // sequences add at most one partial chunk each.
  const size_t per_row = ((size_t)T + kChunk - 1) / kChunk;
  L.n_chunks_ub = (N == B && B > 1) ? (size_t)B * per_row : per_row + (size_t)N;
  // bf16 inputs run the fused kernel, which needs only the sequence table.
  L.rec_bytes = in_dtype == CKDA_F32 ? f64_record_bytes(dk, dv) : 0;
  L.total = L.table_bytes + L.n_chunks_ub * (size_t)H * L.rec_bytes;
  return L;
}

// Backward workspace: the sequence table, then per (chunk, head) the fp64
// record, the state entering the chunk, U, dU, the state gradient at the
// chunk's end and the per-chunk scratch, each region 256-byte aligned.
struct BwdLayout {
  size_t table, rec_bytes, n_chunks_ub;
  size_t records, S, U, dU, dSe, scratch, total;   // byte offsets, then the total
};

static BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, int N) {
  BwdLayout L{};
  const FwdLayout F = fwd_layout(B, T, H, dk, dv, N, CKDA_F32);
  const size_t ch = F.n_chunks_ub * (size_t)H;
  L.n_chunks_ub = F.n_chunks_ub;
  L.rec_bytes = F.rec_bytes;
  L.table = F.table_bytes;
  L.records = L.table;
  L.S = L.records + align256(ch * L.rec_bytes);
  L.U = L.S + align256(ch * dk * dv * sizeof(double));
  L.dU = L.U + align256(ch * kChunk * dv * sizeof(double));
  L.dSe = L.dU + align256(ch * kChunk * dv * sizeof(double));
  L.scratch = L.dSe + align256(ch * dk * dv * sizeof(double));
  L.total = L.scratch + align256(ch * f64_bwd_scratch_bytes(dk, dv));
  return L;
}

SeqTable seq_table(void *workspace, int N) {
  int32_t *base = static_cast<int32_t *>(workspace);
  SeqTable t;
  t.seq_start = base;
  t.seq_len = base + N;
  t.chunk_off = base + 2 * (size_t)N;
  t.order = base + 3 * (size_t)N + 1;
  return t;
}

}  // namespace ckda

using namespace ckda;

namespace {

bool dims_ok(int d) { return d == 64 || d == 128; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int forward_shape_status(int B, int T, int H, int dk, int dv, int N, int in_dtype,
                         bool packed) {
  if (in_dtype != CKDA_BF16 && in_dtype != CKDA_F32) return CKDA_ERR_DTYPE;
  if (B < 1 || T < 0 || H < 1 || N < 1 || !dims_ok(dk) || !dims_ok(dv)) return CKDA_ERR_SHAPE;
  if ((long long)B * T * H >= (1LL << 31)) return CKDA_ERR_SHAPE;
  if ((long long)N * H >= (1LL << 31)) return CKDA_ERR_SHAPE;
  // The kernels address one chunk of one head's rows with 32-bit byte offsets:
  // 64 token rows of H heads at up to max(dk, dv) fp32 values each.
  if ((long long)H * (dk > dv ? dk : dv) * 4 * kChunk >= (1LL << 31)) return CKDA_ERR_SHAPE;
  if (packed ? B != 1 : N != B) return CKDA_ERR_SHAPE;
  return CKDA_OK;
}

bool debug_mode() {
  const char *e = getenv("CKDA_DEBUG");
  return e && *e && strcmp(e, "0") != 0;
}

// Debug mode: the host copy of cu_seqlens must be non-decreasing from 0 to T.
// Copied in pieces through a stack buffer, so the check allocates nothing.
int debug_check_cu(const int32_t *cu_seqlens, int N, int T, hipStream_t st) {
  constexpr int kPiece = 256;
  int32_t h[kPiece];
  int32_t prev = 0;
  for (int i0 = 0; i0 <= N; i0 += kPiece) {
    const int n = (N + 1 - i0) < kPiece ? (N + 1 - i0) : kPiece;
    if (hipMemcpyAsync(h, cu_seqlens + i0, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost,
                       st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return CKDA_ERR_LAUNCH;
    for (int i = 0; i < n; ++i) {
      if ((i0 + i == 0 && h[i] != 0) || h[i] < prev) return CKDA_ERR_SHAPE;
      prev = h[i];
    }
  }
  return prev == T ? CKDA_OK : CKDA_ERR_SHAPE;
}

// Debug-mode steps shared by the forward and the backward, after validation.
int debug_prologue(const int32_t *cu_seqlens, int N, int T, void *workspace, size_t bytes,
                   hipStream_t st) {
  if (!debug_mode()) return CKDA_OK;
  if (cu_seqlens)
    if (int s = debug_check_cu(cu_seqlens, N, T, st)) return s;
  if (workspace && launch_poison(workspace, bytes & ~(size_t)3, st) != hipSuccess)
    return CKDA_ERR_LAUNCH;
  return CKDA_OK;
}

}  // namespace

extern "C" int ckda_abi_version(void) { return 1; }

extern "C" const char *ckda_status_string(int status) {
  switch (status) {
    case CKDA_OK: return "ok";
    case CKDA_ERR_NULL: return "a required pointer is NULL";
    case CKDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case CKDA_ERR_DTYPE: return "unknown input dtype";
    case CKDA_ERR_ALIGN: return "a device pointer is misaligned";
    case CKDA_ERR_WORKSPACE: return "workspace missing or too small";
    case CKDA_ERR_LAUNCH: return "kernel launch failed";
    case CKDA_ERR_ALIAS: return "an output overlaps an input it may not alias";
    case CKDA_ERR_SCRATCH:
      return "the call needs more scratch than the fixed no-allocation buffer holds";
    default: return "unknown status";
  }
}

extern "C" size_t ckda_forward_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                               int in_dtype) {
  // The layout does not depend on packing; accept either form of N.
  if (forward_shape_status(B, T, H, dk, dv, N, in_dtype, B == 1 && N != B) != CKDA_OK)
    return 0;
  return fwd_layout(B, T, H, dk, dv, N, in_dtype).total;
}

namespace {

// Workspace of a forward with these options: the layout above, then (with
// CKDA_OPT_SPLIT) the slot images of the two-kernel hand-off.
size_t forward_ex_bytes(int B, int T, int H, int dk, int dv, int N, int in_dtype, int options) {
  const size_t base = fwd_layout(B, T, H, dk, dv, N, in_dtype).total;
  if (!(options & CKDA_OPT_SPLIT)) return base;
  return align256(base) + fwd_bf16_split_bytes(T, H, dk, N);
}

}  // namespace

extern "C" size_t ckda_forward_ex_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                  int in_dtype, int options) {
  if (forward_shape_status(B, T, H, dk, dv, N, in_dtype, B == 1 && N != B) != CKDA_OK)
    return 0;
  return forward_ex_bytes(B, T, H, dk, dv, N, in_dtype, options);
}

namespace {

int forward_impl(const void *q, const void *k, const void *v, const float *g, const float *beta,
                 const float *S0, const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                 int N, int in_dtype, int options, void *o, float *S_T, void *workspace,
                 size_t workspace_bytes, void *stream) {
  const bool packed = cu_seqlens != nullptr;
  if (int s = forward_shape_status(B, T, H, dk, dv, N, in_dtype, packed)) return s;
  if (options & ~(CKDA_OPT_KDA | CKDA_OPT_QK_L2NORM | CKDA_OPT_O_BF16 | CKDA_OPT_SPLIT))
    return CKDA_ERR_SHAPE;
  const int signed_gates = (options & CKDA_OPT_KDA) ? 0 : 1;
  const int l2norm = (options & CKDA_OPT_QK_L2NORM) ? 1 : 0;
  const int o_bf16 = (options & CKDA_OPT_O_BF16) ? 1 : 0;
  const bool split = (options & CKDA_OPT_SPLIT) != 0;
  if (split && (in_dtype != CKDA_BF16 || packed || l2norm || o_bf16)) return CKDA_ERR_SHAPE;
  const size_t rows = (size_t)B * T * H;
  if (rows > 0 && (!q || !k || !v || !g || !beta || !o)) return CKDA_ERR_NULL;
  const void *ptrs[] = {q, k, v, g, S0, o, S_T, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return CKDA_ERR_ALIGN;
  if ((beta && !aligned4(beta)) || (cu_seqlens && !aligned4(cu_seqlens))) return CKDA_ERR_ALIGN;

  const size_t in_sz = in_dtype == CKDA_BF16 ? 2 : 4;
  const size_t st_bytes = (size_t)N * H * dk * dv * 4;
  const size_t o_bytes = rows * dv * (o_bf16 ? 2 : 4);
  struct Span { const void *p; size_t n; };
  const Span ins[] = {{q, rows * dk * in_sz}, {k, rows * dk * in_sz}, {v, rows * dv * in_sz},
                      {g, rows * dk * 4},      {beta, rows * 4},       {cu_seqlens, ((size_t)N + 1) * 4}};
  for (const Span &s : ins) {
    if (overlaps(o, o_bytes, s.p, s.n)) return CKDA_ERR_ALIAS;
    if (overlaps(S_T, st_bytes, s.p, s.n)) return CKDA_ERR_ALIAS;
  }
  if (overlaps(o, o_bytes, S0, st_bytes) || overlaps(o, o_bytes, S_T, st_bytes))
    return CKDA_ERR_ALIAS;
  if (S_T != S0 && overlaps(S_T, st_bytes, S0, st_bytes)) return CKDA_ERR_ALIAS;

  const FwdLayout L = fwd_layout(B, T, H, dk, dv, N, in_dtype);
  const size_t need = forward_ex_bytes(B, T, H, dk, dv, N, in_dtype, options);
  if (!workspace || workspace_bytes < need) return CKDA_ERR_WORKSPACE;
  if (overlaps(workspace, need, o, o_bytes) || overlaps(workspace, need, S_T, st_bytes) ||
      overlaps(workspace, need, S0, st_bytes))
    return CKDA_ERR_ALIAS;
  for (const Span &s : ins)
    if (overlaps(workspace, need, s.p, s.n)) return CKDA_ERR_ALIAS;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (int s = debug_prologue(cu_seqlens, N, T, workspace, L.total, st)) return s;
  const SeqTable tab = seq_table(workspace, N);
  hipError_t e;
  if (in_dtype == CKDA_BF16) {
    // Uniform rows need no table: the kernel derives each sequence from its row.
    if (packed && launch_seq_table(cu_seqlens, B, T, N, tab, st) != hipSuccess)
      return CKDA_ERR_LAUNCH;
    if (split)
      e = launch_fwd_bf16_split(q, k, v, g, beta, S0, o, S_T, T, H, dk, dv, N, tab, signed_gates,
                                static_cast<char *>(workspace) + align256(L.total), st);
    else
      e = launch_fwd_bf16(q, k, v, g, beta, S0, o, S_T, T, H, dk, dv, N, tab, packed ? 1 : 0,
                          signed_gates, l2norm, o_bf16, st);
  } else {
    if (launch_seq_table(cu_seqlens, B, T, N, tab, st) != hipSuccess) return CKDA_ERR_LAUNCH;
    void *records = static_cast<char *>(workspace) + L.table_bytes;
    e = launch_fwd_f64(q, k, v, g, beta, S0, B * T, H, dk, dv, N, in_dtype, tab, L.n_chunks_ub,
                       records, L.rec_bytes, o, S_T, signed_gates, l2norm, o_bf16, st);
  }
  return e == hipSuccess ? CKDA_OK : CKDA_ERR_LAUNCH;
}

}  // namespace

extern "C" int ckda_forward(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *S0, const int32_t *cu_seqlens,
                            int B, int T, int H, int dk, int dv, int N, int in_dtype, float *o,
                            float *S_T, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, 0, o, S_T,
                      workspace, workspace_bytes, stream);
}

extern "C" int kda_forward(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, const int32_t *cu_seqlens,
                           int B, int T, int H, int dk, int dv, int N, int in_dtype, float *o,
                           float *S_T, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype,
                      CKDA_OPT_KDA, o, S_T, workspace, workspace_bytes, stream);
}

extern "C" int ckda_forward_ex(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *S0, const int32_t *cu_seqlens,
                               int B, int T, int H, int dk, int dv, int N, int in_dtype,
                               int options, void *o, float *S_T, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return forward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, options, o,
                      S_T, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- no allocation
// For callers that cannot allocate (graph capture, tight serving loops): the
// workspace is a fixed file-scope device array.  Host code never passes the
// array's name to a kernel; it uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
namespace {

constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current; NULL if the lookup fails.
void *static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t ckda_forward_noalloc_max_bytes(void) { return kStaticScratchBytes; }

extern "C" int ckda_forward_noalloc(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *S0,
                                    const int32_t *cu_seqlens, int B, int T, int H, int dk,
                                    int dv, int N, int in_dtype, int options, void *o,
                                    float *S_T, void *stream) {
  const bool packed = cu_seqlens != nullptr;
  if (int s = forward_shape_status(B, T, H, dk, dv, N, in_dtype, packed)) return s;
  if (forward_ex_bytes(B, T, H, dk, dv, N, in_dtype, options) > kStaticScratchBytes)
    return CKDA_ERR_SCRATCH;
  void *ws = static_scratch();
  if (!ws) return CKDA_ERR_LAUNCH;
  return forward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, options,
                      o, S_T, ws, kStaticScratchBytes, stream);
}

extern "C" size_t ckda_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                int in_dtype) {
  if (forward_shape_status(B, T, H, dk, dv, N, in_dtype, B == 1 && N != B) != CKDA_OK) return 0;
  return bwd_layout(B, T, H, dk, dv, N).total;
}

namespace {

int backward_impl(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const float *S0, const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                  int N, int in_dtype, const float *d_o, const float *dS_T, float *dq,
                  float *dk_out, float *dv_out, float *dg, float *dbeta, float *dS0,
                  void *workspace, size_t workspace_bytes, int options, void *stream) {
  const bool packed = cu_seqlens != nullptr;
  if (int s = forward_shape_status(B, T, H, dk, dv, N, in_dtype, packed)) return s;
  if (options & ~(CKDA_OPT_KDA | CKDA_OPT_QK_L2NORM)) return CKDA_ERR_SHAPE;
  const int signed_gates = (options & CKDA_OPT_KDA) ? 0 : 1;
  const int l2norm = (options & CKDA_OPT_QK_L2NORM) ? 1 : 0;
  const size_t rows = (size_t)B * T * H;
  if (rows > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk_out || !dv_out || !dg ||
                   !dbeta))
    return CKDA_ERR_NULL;
  const void *ptrs[] = {q, k, v, g, S0, d_o, dS_T, dq, dk_out, dv_out, dg, dS0, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return CKDA_ERR_ALIGN;
  if ((beta && !aligned4(beta)) || (dbeta && !aligned4(dbeta)) ||
      (cu_seqlens && !aligned4(cu_seqlens)))
    return CKDA_ERR_ALIGN;

  const size_t in_sz = in_dtype == CKDA_BF16 ? 2 : 4;
  const size_t st_bytes = (size_t)N * H * dk * dv * 4;
  const BwdLayout L = bwd_layout(B, T, H, dk, dv, N);
  struct Span { const void *p; size_t n; };
  const Span ins[] = {{q, rows * dk * in_sz}, {k, rows * dk * in_sz}, {v, rows * dv * in_sz},
                      {g, rows * dk * 4},      {beta, rows * 4},       {S0, st_bytes},
                      {cu_seqlens, ((size_t)N + 1) * 4}, {d_o, rows * dv * 4}, {dS_T, st_bytes}};
  const Span outs[] = {{dq, rows * dk * 4}, {dk_out, rows * dk * 4}, {dv_out, rows * dv * 4},
                       {dg, rows * dk * 4}, {dbeta, rows * 4},       {dS0, st_bytes},
                       {workspace, L.total}};
  const int n_outs = sizeof(outs) / sizeof(outs[0]);
  for (int a = 0; a < n_outs; ++a) {
    for (const Span &s : ins)
      if (overlaps(outs[a].p, outs[a].n, s.p, s.n)) return CKDA_ERR_ALIAS;
    for (int b = a + 1; b < n_outs; ++b)
      if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return CKDA_ERR_ALIAS;
  }
  if (!workspace || workspace_bytes < L.total) return CKDA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (int s = debug_prologue(cu_seqlens, N, T, workspace, L.total, st)) return s;
  const SeqTable tab = seq_table(workspace, N);
  if (launch_seq_table(cu_seqlens, B, T, N, tab, st) != hipSuccess) return CKDA_ERR_LAUNCH;
  char *w = static_cast<char *>(workspace);
  hipError_t e = launch_bwd_f64(
      q, k, v, g, beta, S0, d_o, dS_T, H, dk, dv, N, in_dtype, tab, L.n_chunks_ub,
      w + L.records, L.rec_bytes, reinterpret_cast<double *>(w + L.S),
      reinterpret_cast<double *>(w + L.U), reinterpret_cast<double *>(w + L.dU),
      reinterpret_cast<double *>(w + L.dSe), reinterpret_cast<double *>(w + L.scratch), dq,
      dk_out, dv_out, dg, dbeta, dS0, signed_gates, l2norm, st);
  return e == hipSuccess ? CKDA_OK : CKDA_ERR_LAUNCH;
}

}  // namespace

extern "C" int ckda_backward(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *S0, const int32_t *cu_seqlens,
                             int B, int T, int H, int dk, int dv, int N, int in_dtype,
                             const float *d_o, const float *dS_T, float *dq, float *dk_out,
                             float *dv_out, float *dg, float *dbeta, float *dS0, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return backward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, d_o, dS_T,
                       dq, dk_out, dv_out, dg, dbeta, dS0, workspace, workspace_bytes, 0, stream);
}

extern "C" int ckda_backward_ex(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *S0, const int32_t *cu_seqlens,
                                int B, int T, int H, int dk, int dv, int N, int in_dtype,
                                int options, const float *d_o, const float *dS_T, float *dq,
                                float *dk_out, float *dv_out, float *dg, float *dbeta,
                                float *dS0, void *workspace, size_t workspace_bytes,
                                void *stream) {
  return backward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, d_o, dS_T,
                       dq, dk_out, dv_out, dg, dbeta, dS0, workspace, workspace_bytes, options,
                       stream);
}

extern "C" int kda_backward(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *S0, const int32_t *cu_seqlens,
                            int B, int T, int H, int dk, int dv, int N, int in_dtype,
                            const float *d_o, const float *dS_T, float *dq, float *dk_out,
                            float *dv_out, float *dg, float *dbeta, float *dS0, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return backward_impl(q, k, v, g, beta, S0, cu_seqlens, B, T, H, dk, dv, N, in_dtype, d_o, dS_T,
                       dq, dk_out, dv_out, dg, dbeta, dS0, workspace, workspace_bytes, CKDA_OPT_KDA,
                       stream);
}

extern "C" int ckda_decode_step(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, float *S, float *o, int N, int H, int dk,
                                int dv, int in_dtype, void *stream) {
  if (in_dtype != CKDA_BF16 && in_dtype != CKDA_F32) return CKDA_ERR_DTYPE;
  if (N < 1 || H < 1 || !dims_ok(dk) || !dims_ok(dv)) return CKDA_ERR_SHAPE;
  if ((long long)N * H >= (1LL << 31)) return CKDA_ERR_SHAPE;
  if (!q || !k || !v || !g || !beta || !S || !o) return CKDA_ERR_NULL;
  const void *ptrs[] = {q, k, v, g, S, o};
  for (const void *p : ptrs)
    if (!aligned16(p)) return CKDA_ERR_ALIGN;
  if (!aligned4(beta)) return CKDA_ERR_ALIGN;
  const size_t nh = (size_t)N * H;
  const size_t in_sz = in_dtype == CKDA_BF16 ? 2 : 4;
  const size_t s_bytes = nh * dk * dv * 4, o_bytes = nh * dv * 4;
  struct Span { const void *p; size_t n; };
  const Span ins[] = {{q, nh * dk * in_sz}, {k, nh * dk * in_sz}, {v, nh * dv * in_sz},
                      {g, nh * dk * 4},     {beta, nh * 4}};
  if (overlaps(o, o_bytes, S, s_bytes)) return CKDA_ERR_ALIAS;
  for (const Span &s : ins)
    if (overlaps(S, s_bytes, s.p, s.n) || overlaps(o, o_bytes, s.p, s.n)) return CKDA_ERR_ALIAS;
  hipError_t e = launch_decode(q, k, v, g, beta, S, o, N, H, dk, dv, in_dtype,
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CKDA_OK : CKDA_ERR_LAUNCH;
}
