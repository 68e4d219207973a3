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
