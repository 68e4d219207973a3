/*
 * CPU oracle for the Complex KDA (CKDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code with the HIP library.
 *
 * What it computes (plain definition, token by token, in fp64):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t                     (readout after token t's update)
 *
 * The update rule is the one printed in the blog post "One update, one
 * quarter turn" (section "ELI5: the whiteboard, the mirror, and the clock",
 * paragraph "The mirror"): read right to left it decays the old state by the
 * per-channel gate alpha, erases along the key direction k, and writes the
 * outer product k v^T.  The state S is dk x dv; the gate scales its rows (key
 * channels).  The readout S_t^T q_t is not printed on any page; it is the
 * usual linear-attention read of the state after the write.
 *
 * The erase-and-write step is applied in the algebraically identical form
 *   S <- Diag(alpha) S;  u = S^T k;  S <- S + beta k (v - u)^T
 * which is (I - beta k k^T) S' + beta k v^T with S' = Diag(alpha) S.
 *
 * Gate range: the CKDA paper ("Complex KDA", ai.info summary, sections
 * "What This Paper Is About" and the authors' abstract) extends alpha to
 * [-1, 1] and beta to [0, 2].  The oracle accepts any finite value and
 * computes the definition as written; it applies no clamp.
 *
 * Parallelism: independent (sequence, head) pairs are spread over POSIX
 * threads.  Within a pair the tokens run strictly in order.
 *
 * ckda_oracle_backward is the reverse-mode gradient of the same recurrence
 * (its comment gives the adjoint steps); it is a plain application of the
 * chain rule to the four token operations above, run from the last token to
 * the first.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *S0;
    const int64_t *starts;   /* token offset of each sequence (row of [*,H,*]) */
    const int64_t *lens;     /* length of each sequence */
    int H, dk, dv, N;
    double *o, *S_T;
    int next;                /* next (sequence, head) job, guarded by mu */
    pthread_mutex_t mu;
} fwd_job;

/* One (sequence, head) pair: run the recurrence over its tokens. */
static void run_pair(const fwd_job *J, int n, int h, double *S, double *u) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const size_t sz = (size_t)dk * dv;
    if (J->S0)
        memcpy(S, J->S0 + ((size_t)n * H + h) * sz, sz * sizeof(double));
    else
        memset(S, 0, sz * sizeof(double));

    for (int64_t s = 0; s < J->lens[n]; ++s) {
        const size_t row = (size_t)(J->starts[n] + s) * H + h; /* token-head row */
        const double *q = J->q + row * dk, *k = J->k + row * dk;
        const double *v = J->v + row * dv, *a = J->g + row * dk;
        const double b = J->beta[row];
        double *o = J->o + row * dv;

        /* decay: S <- Diag(alpha) S (gate scales row c, the key channel) */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= a[c];
        /* u = S^T k */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) u[j] += k[c] * S[c * dv + j];
        /* erase along k and write k v^T: S <- S + beta k (v - u)^T */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] += b * k[c] * (v[j] - u[j]);
        /* readout o = S^T q */
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) o[j] += q[c] * S[c * dv + j];
    }
    if (J->S_T) memcpy(J->S_T + ((size_t)n * H + h) * sz, S, sz * sizeof(double));
}

static void *fwd_worker(void *arg) {
    fwd_job *J = (fwd_job *)arg;
    double *S = (double *)malloc((size_t)J->dk * J->dv * sizeof(double));
    double *u = (double *)malloc((size_t)J->dv * sizeof(double));
    if (!S || !u) { free(S); free(u); return NULL; }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int p = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (p >= J->N * J->H) break;
        run_pair(J, p / J->H, p % J->H, S, u);
    }
    free(S);
    free(u);
    return NULL;
}

/*
 * Forward over N sequences.
 *
 *  q, k, g : [rows, H, dk]   v, o : [rows, H, dv]   beta : [rows, H]
 *  S0, S_T : [N, H, dk, dv]  (S0 == NULL: zero state; S_T == NULL: not written)
 *  cu_seqlens : NULL  -> N = B sequences of length T, rows = B*T
 *               else  -> N+1 offsets into rows (B must be 1, rows = T)
 *  All floating-point buffers are host fp64.  Returns 0, or -1 on bad sizes.
 */
int ckda_oracle_forward(const double *q, const double *k, const double *v,
                        const double *g, const double *beta, const double *S0,
                        const int64_t *cu_seqlens, int B, int T, int H, int dk,
                        int dv, int N, double *o, double *S_T, int nthreads) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0) return -1;
    if (cu_seqlens && B != 1) return -1;
    if (!cu_seqlens && N != B) return -1;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    int64_t *lens = (int64_t *)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    if (!starts || !lens) { free(starts); free(lens); return -1; }
    for (int n = 0; n < N; ++n) {
        if (cu_seqlens) {
            starts[n] = cu_seqlens[n];
            lens[n] = cu_seqlens[n + 1] - cu_seqlens[n];
            if (lens[n] < 0 || cu_seqlens[n + 1] > T) { free(starts); free(lens); return -1; }
        } else {
            starts[n] = (int64_t)n * T;
            lens[n] = T;
        }
    }
    fwd_job J = {q, k, v, g, beta, S0, starts, lens, H, dk, dv, N, o, S_T, 0,
                 PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > N * H) nthreads = N * H > 0 ? N * H : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    int started = 0;
    for (int i = 0; i < nthreads && tid; ++i)
        if (pthread_create(&tid[i], NULL, fwd_worker, &J) == 0) ++started;
    if (started == 0) fwd_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    free(starts);
    free(lens);
    return 0;
}

/*
 * One decode step for N*H independent states, in place:
 *   S <- (I - beta k k^T) Diag(alpha) S + beta k v^T ;  o = S^T q
 *  q, k, g : [N, H, dk]  v, o : [N, H, dv]  beta : [N, H]  S : [N, H, dk, dv]
 */
int ckda_oracle_decode(const double *q, const double *k, const double *v,
                       const double *g, const double *beta, double *S, double *o,
                       int N, int H, int dk, int dv, int nthreads) {
    /* A decode step is a length-1 forward whose S0 and S_T are the same
       buffer; route it through the same per-pair code. */
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    return ckda_oracle_forward(q, k, v, g, beta, S, NULL, N, 1, H, dk, dv, N, o, S,
                               nthreads);
}

/* ------------------------------------------------------------------ backward
 *
 * Gradient of  L = sum(dO * o) + sum(dS_T * S_T)  with respect to q, k, v,
 * alpha (g), beta and S0, for upstream gradients dO (of every o_t) and dS_T
 * (of the final states; NULL = zero).
 *
 * Per token, with P = S_{t-1} the state before it, the forward computes
 *   S' = Diag(alpha) P;  u = S'^T k;  delta = beta (v - u);
 *   S_t = S' + k delta^T;  o = S_t^T q
 * and the chain rule, applied to these operations from the last to the first,
 * gives (dS holds dL/dS_t on entry and dL/dS_{t-1} on exit):
 *   dS += q dO_t^T            dq = S_t dO_t
 *   ddelta = dS^T k           dk = dS delta
 *   dv = beta ddelta          dbeta = (v - u) . ddelta       du = -beta ddelta
 *   dS += k du^T              dk += S' du                     (dS = dL/dS')
 *   dalpha_c = sum_j dS[c,j] P[c,j]                           dS <- Diag(alpha) dS
 * The states P are recomputed segment by segment from checkpoints taken every
 * kSeg tokens, with the same operations as the forward above, so they are bit
 * for bit the states of the forward pass; only the memory held differs.
 */
enum { kSeg = 64 };

typedef struct {
    const double *q, *k, *v, *g, *beta, *S0, *dO, *dS_T;
    const int64_t *starts, *lens;
    int H, dk, dv, N;
    double *dq, *dk_out, *dv_out, *dg, *dbeta, *dS0;
    int next, failed;
    pthread_mutex_t mu;
} bwd_job;

/* The forward update of one token on S in place; u receives S'^T k. */
static void bwd_recompute_token(const double *k, const double *v, const double *a, double b,
                                double *S, double *u, int dk, int dv) {
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] *= a[c];
    for (int j = 0; j < dv; ++j) u[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) u[j] += k[c] * S[c * dv + j];
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] += b * k[c] * (v[j] - u[j]);
}

static int run_pair_bwd(const bwd_job *J, int n, int h) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const size_t sz = (size_t)dk * dv;
    const int64_t L = J->lens[n];
    const int64_t nseg = (L + kSeg - 1) / kSeg;
    double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg > 0 ? nseg : 1));
    double *pre = (double *)malloc(sizeof(double) * sz * kSeg);
    double *S = (double *)malloc(sizeof(double) * sz);
    double *Sp = (double *)malloc(sizeof(double) * sz);
    double *dS = (double *)malloc(sizeof(double) * sz);
    double *u = (double *)malloc(sizeof(double) * dv);
    double *delta = (double *)malloc(sizeof(double) * dv);
    double *dd = (double *)malloc(sizeof(double) * dv);
    int ok = ck && pre && S && Sp && dS && u && delta && dd;
    if (ok) {
        const size_t pair = (size_t)n * H + h;
        if (J->S0) memcpy(S, J->S0 + pair * sz, sz * sizeof(double));
        else memset(S, 0, sz * sizeof(double));
#define ROW(s) ((size_t)(J->starts[n] + (s)) * H + h)
        /* forward pass, keeping the state at the start of every segment */
        for (int64_t s = 0; s < L; ++s) {
            if (s % kSeg == 0) memcpy(ck + (size_t)(s / kSeg) * sz, S, sz * sizeof(double));
            const size_t r = ROW(s);
            bwd_recompute_token(J->k + r * dk, J->v + r * dv, J->g + r * dk, J->beta[r], S, u,
                                dk, dv);
        }
        if (J->dS_T) memcpy(dS, J->dS_T + pair * sz, sz * sizeof(double));
        else memset(dS, 0, sz * sizeof(double));
        for (int64_t seg = nseg - 1; seg >= 0; --seg) {
            const int64_t s0 = seg * kSeg, s1 = (s0 + kSeg < L) ? s0 + kSeg : L;
            memcpy(S, ck + (size_t)seg * sz, sz * sizeof(double));
            for (int64_t s = s0; s < s1; ++s) {
                memcpy(pre + (size_t)(s - s0) * sz, S, sz * sizeof(double));
                const size_t r = ROW(s);
                bwd_recompute_token(J->k + r * dk, J->v + r * dv, J->g + r * dk, J->beta[r], S,
                                    u, dk, dv);
            }
            for (int64_t s = s1 - 1; s >= s0; --s) {
                const size_t r = ROW(s);
                const double *q = J->q + r * dk, *k = J->k + r * dk, *v = J->v + r * dv;
                const double *a = J->g + r * dk, *dO = J->dO + r * dv;
                const double b = J->beta[r];
                const double *P = pre + (size_t)(s - s0) * sz;
                double *dq = J->dq + r * dk, *dk_ = J->dk_out + r * dk;
                double *dv_ = J->dv_out + r * dv, *dg = J->dg + r * dk;
                /* this token's forward quantities: S', u, delta and S_t (in S) */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) Sp[c * dv + j] = a[c] * P[c * dv + j];
                for (int j = 0; j < dv; ++j) u[j] = 0.0;
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) u[j] += k[c] * Sp[c * dv + j];
                for (int j = 0; j < dv; ++j) delta[j] = b * (v[j] - u[j]);
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) S[c * dv + j] = Sp[c * dv + j] + k[c] * delta[j];
                /* readout o = S_t^T q */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) dS[c * dv + j] += q[c] * dO[j];
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += S[c * dv + j] * dO[j];
                    dq[c] = acc;
                }
                /* S_t = S' + k delta^T */
                for (int j = 0; j < dv; ++j) dd[j] = 0.0;
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) dd[j] += dS[c * dv + j] * k[c];
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dS[c * dv + j] * delta[j];
                    dk_[c] = acc;
                }
                /* delta = beta (v - u) */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dv_[j] = b * dd[j];
                    db += (v[j] - u[j]) * dd[j];
                }
                J->dbeta[r] = db;
                /* u = S'^T k, with du = -beta ddelta */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) dS[c * dv + j] += k[c] * (-b * dd[j]);
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += Sp[c * dv + j] * (-b * dd[j]);
                    dk_[c] += acc;
                }
                /* S' = Diag(alpha) P */
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dS[c * dv + j] * P[c * dv + j];
                    dg[c] = acc;
                }
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) dS[c * dv + j] *= a[c];
            }
        }
#undef ROW
        memcpy(J->dS0 + pair * sz, dS, sz * sizeof(double));
    }
    free(ck); free(pre); free(S); free(Sp); free(dS); free(u); free(delta); free(dd);
    return ok;
}

static void *bwd_worker(void *arg) {
    bwd_job *J = (bwd_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int p = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (p >= J->N * J->H) break;
        if (!run_pair_bwd(J, p / J->H, p % J->H)) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

/*
 * Backward over N sequences; layouts as ckda_oracle_forward.
 *  dO : [rows, H, dv]          dS_T : [N, H, dk, dv] or NULL (zero)
 *  dq, dk, dg : [rows, H, dk]  dv : [rows, H, dv]  dbeta : [rows, H]
 *  dS0 : [N, H, dk, dv]
 * Gradients of rows that belong to no sequence are left untouched.  Returns
 * 0, -1 on bad sizes, -2 if memory ran out.
 */
int ckda_oracle_backward(const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *S0,
                         const int64_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                         int N, const double *dO, const double *dS_T, double *dq,
                         double *dk_out, double *dv_out, double *dg, double *dbeta,
                         double *dS0, int nthreads) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0) return -1;
    if (cu_seqlens && B != 1) return -1;
    if (!cu_seqlens && N != B) return -1;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    int64_t *lens = (int64_t *)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    if (!starts || !lens) { free(starts); free(lens); return -2; }
    for (int n = 0; n < N; ++n) {
        if (cu_seqlens) {
            starts[n] = cu_seqlens[n];
            lens[n] = cu_seqlens[n + 1] - cu_seqlens[n];
            if (lens[n] < 0 || cu_seqlens[n + 1] > T) { free(starts); free(lens); return -1; }
        } else {
            starts[n] = (int64_t)n * T;
            lens[n] = T;
        }
    }
    bwd_job J = {q, k, v, g, beta, S0, dO, dS_T, starts, lens, H, dk, dv, N,
                 dq, dk_out, dv_out, dg, dbeta, dS0, 0, 0, PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > N * H) nthreads = N * H > 0 ? N * H : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    int started = 0;
    for (int i = 0; i < nthreads && tid; ++i)
        if (pthread_create(&tid[i], NULL, bwd_worker, &J) == 0) ++started;
    if (started == 0) bwd_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    free(starts);
    free(lens);
    return J.failed ? -2 : 0;
}
