/*
 * ckda.h -- C ABI of the Complex KDA (CKDA) recurrence library for AMD
 * Instinct MI355X (gfx950).
 *
 * The recurrence (update rule: blog post "One update, one quarter turn",
 * section "ELI5: the whiteboard, the mirror, and the clock", paragraph "The
 * mirror"; gate ranges: "Complex KDA" AI summary, section "What This Paper Is
 * About", and the authors' abstract):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t                       (read after token t's write)
 *
 * S is a dk x dv matrix per (sequence, head); alpha_t is a per-key-channel
 * signed gate (nominally in [-1, 1]) and beta_t a per-token scalar (nominally
 * in [0, 2]).  Values outside those ranges are accepted and computed by the
 * same formulas; beta > 2 is a legitimate setting (the summary's Theorem 5).
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers in one HIP device's memory, owned by
 *    the caller.  The library allocates no
 *    memory, keeps no state between calls, and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *    call returns.  Device faults therefore surface at the caller's next
 *    synchronisation.
 *  - Tensors are dense, row-major (C order), with the shapes given below.
 *    q, k, v, g, states, outputs and the workspace must be 16-byte aligned;
 *    beta and cu_seqlens 4-byte aligned.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns an error status and has no side effect.  The
 *    contents of device buffers (e.g. cu_seqlens) are not inspected on the
 *    host.  Offsets that leave [0, T] or decrease are made monotone on the
 *    device: sequence n covers tokens [P_n, P_{n+1}) with
 *    P_i = min(max(0, cu[0], ..., cu[i]), T), so sequences never overlap and
 *    no access leaves the buffers; rows outside every sequence are not
 *    written.  With the environment variable CKDA_DEBUG set (to anything but
 *    "" or "0") the library instead copies cu_seqlens to the host, which
 *    synchronises the stream, returns CKDA_ERR_SHAPE unless
 *    0 = cu[0] <= ... <= cu[N] = T, and fills the workspace with NaN before
 *    the kernels run.
 *  - Calls that share no output buffer may run concurrently on different
 *    streams.
 *  - A call enqueues kernel launches only (no memset, copy or allocation;
 *    CKDA_DEBUG aside), so it may be captured into a HIP graph on `stream`.
 *    A replay runs the same kernels on the same pointers and sizes and reads
 *    the buffers' contents at replay time.
 */
#ifndef CKDA_H
#define CKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    CKDA_OK = 0,
    CKDA_ERR_NULL = 1,       /* a required pointer is NULL */
    CKDA_ERR_SHAPE = 2,      /* a size is out of range or inconsistent */
    CKDA_ERR_DTYPE = 3,      /* unknown input dtype */
    CKDA_ERR_ALIGN = 4,      /* a device pointer is misaligned (see conventions) */
    CKDA_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required */
    CKDA_ERR_LAUNCH = 6,     /* the HIP runtime refused a kernel launch */
    CKDA_ERR_ALIAS = 7,      /* an output overlaps an input it may not alias */
    CKDA_ERR_SCRATCH = 8     /* ckda_forward_noalloc: the call needs more scratch than
                                its fixed buffer holds */
};

/* Input dtypes for q, k, v.  Gates, beta, states and outputs are fp32. */
enum {
    CKDA_BF16 = 0,           /* q, k, v are bfloat16 */
    CKDA_F32 = 1             /* q, k, v are float32 */
};

/* Options of ckda_forward_ex (bitwise or). */
enum {
    CKDA_OPT_KDA = 1,        /* KDA mode: gate signs ignored (|g| is used) */
    CKDA_OPT_QK_L2NORM = 2,  /* q and k L2-normalised per (token, head) in the kernel */
    CKDA_OPT_O_BF16 = 4,     /* o written as bfloat16 (round to nearest even) */
    CKDA_OPT_SPLIT = 8       /* two-kernel hand-off instead of the fused kernel
                                (kept for measurement; see ckda_forward_ex) */
};

/* Version of this ABI (bumped on any incompatible change). */
int ckda_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *ckda_status_string(int status);

/*
 * Workspace needed by ckda_forward for the same sizes and dtype, in bytes.
 * Depends only on the sizes: a caller may size it once for the largest call.
 * Returns 0 if the sizes are invalid (ckda_forward would return
 * CKDA_ERR_SHAPE for them).
 */
size_t ckda_forward_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                    int in_dtype);

/*
 * Chunkwise-parallel CKDA forward over a batch of sequences.
 *
 * The token recurrence above, computed chunkwise with the WY/UT form of the
 * delta rule: fp32 inputs in chunks of 64 tokens, bf16 inputs with the state
 * stepped every 16 tokens.  Gate signs follow the CKDA summary's methodology
 * (the sign kept apart from the log-space magnitude) wherever the gates'
 * range within a chunk or block needs log space; otherwise the signed gates
 * enter as products.
 *
 *  q, k        [B, T, H, dk]  in_dtype
 *  v           [B, T, H, dv]  in_dtype
 *  g           [B, T, H, dk]  fp32   the signed linear gate alpha (not a log)
 *  beta        [B, T, H]      fp32
 *  S0          [N, H, dk, dv] fp32   initial states, or NULL for zero states
 *  cu_seqlens  NULL: N must equal B; sequence n is row n, T tokens long.
 *              else: int32 [N+1] device array of token offsets into the
 *              T axis (B must be 1): sequence n is tokens
 *              [cu_seqlens[n], cu_seqlens[n+1]); 0 = cu[0] <= ... <= cu[N] = T.
 *              Each sequence starts from its own S0[n] and chunks restart at
 *              every sequence start.
 *  B, T, H     B >= 1, T >= 0, H >= 1 (B*T*H < 2^31, H*max(dk,dv)*256 < 2^31)
 *  dk, dv      each 64 or 128
 *  N           number of sequences (>= 1)
 *  in_dtype    CKDA_BF16 or CKDA_F32
 *  o           [B, T, H, dv]  fp32   output, every token written
 *  S_T         [N, H, dk, dv] fp32   final states, or NULL to skip; may be
 *              the same buffer as S0 (in-place state advance), must not
 *              otherwise overlap an input
 *  workspace   device scratch of at least ckda_forward_workspace_bytes(...)
 *              bytes (may be NULL when that is 0); contents on entry are
 *              ignored and on return are unspecified
 *  stream      hipStream_t to enqueue on
 *
 * Numerics: bf16 inputs run every contraction on bf16 matrix cores with
 * fp32 accumulation, splitting fp32 operands into two bf16 terms (hi + lo)
 * so that products keep ~16 mantissa bits; states and intermediates stay
 * fp32.  fp32 inputs are computed in fp64 and rounded to fp32 on output.
 * Gate magnitudes below 2^-126 are treated as 2^-126 (fp32 inputs: 2^-1000),
 * and so is a NaN gate (the clamp of log2|alpha| to that floor keeps the
 * floor).  A NaN anywhere else reaches only the outputs of its own
 * (sequence, head).
 */
int ckda_forward(const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *S0, const int32_t *cu_seqlens,
                 int B, int T, int H, int dk, int dv, int N, int in_dtype,
                 float *o, float *S_T, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * KDA mode of the same forward: the recurrence with non-negative gates, the
 * baseline the CKDA summary measures its kernel throughput against (section
 * "Main Findings", throughput bullet; KDA keeps alpha in [0, 1]).  The sign
 * of every gate is ignored: |g| is used, so the sign bookkeeping of
 * ckda_forward is skipped.  For gates that are all >= 0 the two entry points
 * compute the same recurrence.  Arguments, layouts, workspace, ownership,
 * aliasing rules and errors are exactly those of ckda_forward.
 */
int kda_forward(const void *q, const void *k, const void *v, const float *g,
                const float *beta, const float *S0, const int32_t *cu_seqlens,
                int B, int T, int H, int dk, int dv, int N, int in_dtype,
                float *o, float *S_T, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * ckda_forward with the pre- and post-processing a layer otherwise does in
 * separate passes over HBM, fused into the same kernels (the CKDA summary's
 * methodology names a variant that fuses the gate signs into the key/query
 * normalisation):
 *
 *  options  0, or any bitwise or of
 *    CKDA_OPT_KDA        as kda_forward
 *    CKDA_OPT_QK_L2NORM  each (token, head) row of q and of k is replaced by
 *                        x * (sum_c x_c^2 + 1e-6)^(-1/2) before use, computed
 *                        in fp32 (bf16 inputs) or fp64 (fp32 inputs); the
 *                        caller's arrays are not modified
 *    CKDA_OPT_O_BF16     o is [B, T, H, dv] bfloat16: the fp32 result rounded
 *                        to nearest even (halves o's HBM traffic)
 *    CKDA_OPT_SPLIT      the chunk preparation as its own kernel: it writes
 *                        every prepared 16-token block (operand planes, T, P,
 *                        gate factors; about 1.8 KB per token and head) to
 *                        the workspace, and a second kernel runs the state
 *                        pass on them.  The same arithmetic as the fused
 *                        kernel, so the results are bit-identical; kept to
 *                        measure that hand-off against the fused kernel.
 *                        bf16 inputs and uniform rows (cu_seqlens NULL) only,
 *                        without CKDA_OPT_QK_L2NORM or CKDA_OPT_O_BF16
 *                        (CKDA_ERR_SHAPE otherwise); the workspace must hold
 *                        ckda_forward_ex_workspace_bytes(...) bytes
 *  o        fp32 or bf16 per CKDA_OPT_O_BF16; 16-byte aligned
 *
 * Every other argument, the workspace size (but for CKDA_OPT_SPLIT) and all
 * error rules are those of ckda_forward; unknown option bits return
 * CKDA_ERR_SHAPE.  ckda_forward is ckda_forward_ex with options 0,
 * kda_forward with CKDA_OPT_KDA.
 */
int ckda_forward_ex(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, const float *S0, const int32_t *cu_seqlens,
                    int B, int T, int H, int dk, int dv, int N, int in_dtype, int options,
                    void *o, float *S_T, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Workspace needed by ckda_forward_ex (and, for its fixed scratch, by
 * ckda_forward_noalloc) with these options, in bytes: that of ckda_forward,
 * plus with CKDA_OPT_SPLIT the hand-off's prepared blocks.  Returns 0 if the
 * sizes are invalid.
 */
size_t ckda_forward_ex_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                       int in_dtype, int options);

/*
 * ckda_forward_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It takes no workspace: the library keeps one fixed scratch array of
 * ckda_forward_noalloc_max_bytes() bytes (64 MiB) per GPU, in device memory
 * that stays held until the process ends, and the call itself allocates
 * nothing (host or device).  Every other argument, layout, option and error
 * is that of ckda_forward_ex; the results are bit-identical to it.
 *
 *  Returns CKDA_ERR_SCRATCH when ckda_forward_ex_workspace_bytes(...) for
 *  the call exceeds the fixed size (bf16 inputs need only a sequence table of
 *  16 bytes per sequence; fp32 inputs need their per-chunk records, and
 *  CKDA_OPT_SPLIT its prepared blocks, so only small such calls fit).
 *
 *  Concurrency: all calls on one GPU share that GPU's scratch, which keeps
 *  the last call's contents (nothing in it needs to start at zero).  Calls
 *  that overlap in time on one GPU -- on different streams, or from
 *  different host threads without ordering -- race on it and give undefined
 *  results; order them on one stream.
 */
int ckda_forward_noalloc(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *S0, const int32_t *cu_seqlens,
                         int B, int T, int H, int dk, int dv, int N, int in_dtype,
                         int options, void *o, float *S_T, void *stream);

/* Size in bytes of the fixed scratch array ckda_forward_noalloc uses. */
size_t ckda_forward_noalloc_max_bytes(void);

/*
 * Workspace needed by ckda_backward for the same sizes, in bytes (the same for
 * both input dtypes).  Returns 0 if the sizes are invalid.  It holds fp64
 * per-chunk intermediates: about 1.3 MB per (64-token chunk, head) at
 * dk = dv = 128.
 */
size_t ckda_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                     int in_dtype);

/*
 * Backward of ckda_forward: the gradient of
 *
 *   L = sum(d_o * o) + sum(dS_T * S_T)
 *
 * with respect to every input, for the upstream gradients d_o (of o) and dS_T
 * (of the final states).  The pages benchmark CKDA's kernels forward plus
 * backward (CKDA summary, "Main Findings", throughput bullet); the gradient is
 * that of the recurrence above, taken by reverse mode through the chunkwise
 * form.  The gate gradient is with respect to the signed alpha itself; gate
 * signs carry no gradient (alpha enters through log|alpha| and its sign).
 *
 *  q .. N, in_dtype    exactly as for ckda_forward (same layouts; the forward
 *                      is recomputed internally, nothing from it is needed)
 *  d_o         [B, T, H, dv]  fp32
 *  dS_T        [N, H, dk, dv] fp32, or NULL for zero
 *  dq, d_k    [B, T, H, dk]  fp32 outputs (gradients of q and k)
 *  d_v         [B, T, H, dv]  fp32 output
 *  dg          [B, T, H, dk]  fp32 output: dL/dalpha
 *  dbeta       [B, T, H]      fp32 output
 *  dS0         [N, H, dk, dv] fp32 output, or NULL to skip
 *  workspace   at least ckda_backward_workspace_bytes(...) bytes of device
 *              scratch; contents on entry ignored, on return unspecified
 *
 * No output may overlap an input, another output or the workspace
 * (CKDA_ERR_ALIAS).  Numerics: every step runs in fp64 (inputs widen
 * exactly) and each gradient is rounded once to fp32.  A gate of exactly 0 is
 * differentiated at |alpha| = 2^-1000, the floor of its log-magnitude, so
 * its own gradient is not meaningful.  ckda_backward_ex below covers the
 * KDA and L2-normalisation options of ckda_forward_ex.
 */
int ckda_backward(const void *q, const void *k, const void *v, const float *g,
                  const float *beta, const float *S0, const int32_t *cu_seqlens,
                  int B, int T, int H, int dk, int dv, int N, int in_dtype,
                  const float *d_o, const float *dS_T, float *dq, float *d_k, float *d_v,
                  float *dg, float *dbeta, float *dS0, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * Backward of kda_forward (KDA mode: gate signs ignored, |g| used), the
 * baseline of the CKDA summary's forward-plus-backward throughput comparison
 * ("Main Findings", throughput bullet).  The loss depends on g only through
 * log|g|, so dg = dlog|g| / g as in ckda_backward.  Arguments, layouts,
 * workspace, aliasing rules and errors are exactly those of ckda_backward.
 */
int kda_backward(const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *S0, const int32_t *cu_seqlens,
                 int B, int T, int H, int dk, int dv, int N, int in_dtype,
                 const float *d_o, const float *dS_T, float *dq, float *d_k, float *d_v,
                 float *dg, float *dbeta, float *dS0, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * ckda_backward with options (bitwise or), the backward of ckda_forward_ex
 * for the same options (the CKDA summary's methodology names Triton kernels
 * that fuse the signs into the key/query normalisation and its backward pass):
 *    0                   as ckda_backward
 *    CKDA_OPT_KDA        as kda_backward
 *    CKDA_OPT_QK_L2NORM  q and k were L2-normalised per (token, head) in the
 *                        forward: x -> x (sum_c x_c^2 + 1e-6)^(-1/2).  dq and
 *                        dk are the gradients with respect to the caller's
 *                        raw q and k, through that normalisation (in fp64)
 * CKDA_OPT_O_BF16 and unknown bits return CKDA_ERR_SHAPE.  Every other
 * argument, the workspace and all error rules are those of ckda_backward.
 */
int ckda_backward_ex(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *S0, const int32_t *cu_seqlens,
                     int B, int T, int H, int dk, int dv, int N, int in_dtype, int options,
                     const float *d_o, const float *dS_T, float *dq, float *d_k, float *d_v,
                     float *dg, float *dbeta, float *dS0, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for N*H independent states, in place.
 *
 *   S <- (I - beta k k^T) Diag(alpha) S + beta k v^T ;  o = S^T q
 *
 *  q, k        [N, H, dk]     in_dtype
 *  v           [N, H, dv]     in_dtype
 *  g           [N, H, dk]     fp32 signed gate alpha
 *  beta        [N, H]         fp32
 *  S           [N, H, dk, dv] fp32, read and overwritten with the new state
 *  o           [N, H, dv]     fp32 output (must not overlap S)
 *  N, H >= 1; dk, dv each 64 or 128; in_dtype CKDA_BF16 or CKDA_F32.
 *
 * Numerics: fp32 throughout (one step adds one rounding per state entry).
 */
int ckda_decode_step(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, float *S, float *o, int N, int H, int dk,
                     int dv, int in_dtype, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CKDA_H */
