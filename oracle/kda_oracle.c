/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64, token-by-token CPU implementation of the Kimi Delta
 * Attention (KDA) recurrence. It is the reference the HIP library is checked
 * against; it shares no code, header or constant with that library. Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * What it computes (per sequence n and value head hv, q/k head h = hv / (HV/H)):
 *
 *     S <- initial_state[n, hv]            (zeros when no initial state is given)
 *     for each token t of sequence n, in order:
 *         S[d, :] *= 2^g[t, hv, d]                 decay first, per key channel d
 *         p        = sum_d k[t, h, d] * S[d, :]     what the state predicts for key k_t
 *         delta    = beta[t, hv] * (v[t, hv, :] - p)
 *         S[d, :] += k[t, h, d] * delta             erase the old value, write the new
 *         o[t, hv, :] = scale * sum_d q[t, h, d] * S[d, :]   read the updated state
 *     final_state[n, hv] = S
 *
 * Sources (the pages): the recurrence is the gated delta rule with per-channel
 * base-2 gates as stated for KDA in "kernel-fun 0.2.0.dev1 sdist, ALGORITHM.md"
 * (intro: all logs base 2, gates <= 0; q/k head h = hv // (HV//H); scale K^-0.5).
 * The order "decay, then erase+write, then read the updated state" is the one the
 * chunk algebra of that page implies: Aqk includes the diagonal i >= j (Stage 2)
 * and o_c = scale*qg@h + Aqk@v' (Stage 3+4). The per-token variant with a per-token
 * log2 gate, 1/sqrt(K) scale and fp32 state per logical sequence is the contract of
 * "Add fused recurrent_kda for decode and inference prefill" (attention-gym PR #317,
 * description): packed int32 offsets, repeated offsets are empty slots whose state
 * passes through bitwise, rows beyond the terminal offset are outside the contract.
 *
 * Layouts (all row-major, last index fastest):
 *   q, k  [B, T, H, K]     v [B, T, HV, V]     g [B, T, HV, K]    beta [B, T, HV]
 *   initial_state / final_state [N, HV, K, V]  (N = B when cu_seqlens is NULL)
 *   o     [B, T, HV, V]
 * Packed mode (cu_seqlens != NULL): B must be 1 and sequence n is tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1 of row 0.
 *
 * Rows of o that belong to no sequence are not written. An empty sequence copies
 * its initial state (or zeros) to final_state with no arithmetic.
 *
 * Threads: one task per (n, hv) chain, taken from a shared counter. Each chain is
 * computed in a fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_BAD_ARGS (-1)
#define KDA_ORACLE_BAD_CU_SEQLENS (-2)
#define KDA_ORACLE_NO_MEMORY (-3)

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0;
    const int32_t *cu;
    double *o, *ht;
    int B, T, H, HV, K, V, N;
    double scale;
    long next;      /* next chain index to take (shared counter) */
    int failed;
    pthread_mutex_t lock;
} job_t;

/* One (sequence, value-head) chain, token by token. */
static int run_chain(job_t *J, long chain, double *S, double *p, double *delta)
{
    const int K = J->K, V = J->V, H = J->H, HV = J->HV, T = J->T;
    const int n = (int)(chain / HV);
    const int hv = (int)(chain % HV);
    const int h = hv / (HV / H);             /* GVA: HV/H value heads share one q/k head */
    long row0, bos, eos;                     /* token rows are (row0 + t) */

    if (J->cu) {
        row0 = 0;
        bos = J->cu[n];
        eos = J->cu[n + 1];
    } else {
        row0 = (long)n * T;
        bos = 0;
        eos = T;
    }

    double *hs = J->ht ? J->ht + ((size_t)n * HV + hv) * (size_t)K * V : NULL;
    const double *h0s = J->h0 ? J->h0 + ((size_t)n * HV + hv) * (size_t)K * V : NULL;

    if (h0s)
        memcpy(S, h0s, sizeof(double) * (size_t)K * V);
    else
        memset(S, 0, sizeof(double) * (size_t)K * V);

    for (long t = bos; t < eos; ++t) {
        const size_t r = (size_t)(row0 + t);
        const double *qt = J->q + (r * H + h) * K;
        const double *kt = J->k + (r * H + h) * K;
        const double *vt = J->v + (r * HV + hv) * V;
        const double *gt = J->g + (r * HV + hv) * K;
        const double bt = J->beta[r * HV + hv];
        double *ot = J->o + (r * HV + hv) * V;

        /* decay: row d of the state is scaled by 2^g[d] */
        for (int d = 0; d < K; ++d) {
            const double a = exp2(gt[d]);
            for (int c = 0; c < V; ++c)
                S[(size_t)d * V + c] *= a;
        }
        /* prediction p = S^T k */
        for (int c = 0; c < V; ++c)
            p[c] = 0.0;
        for (int d = 0; d < K; ++d)
            for (int c = 0; c < V; ++c)
                p[c] += kt[d] * S[(size_t)d * V + c];
        /* correction delta = beta (v - p) */
        for (int c = 0; c < V; ++c)
            delta[c] = bt * (vt[c] - p[c]);
        /* rank-one update S += k delta^T */
        for (int d = 0; d < K; ++d)
            for (int c = 0; c < V; ++c)
                S[(size_t)d * V + c] += kt[d] * delta[c];
        /* read-out from the updated state: o = scale S^T q */
        for (int c = 0; c < V; ++c) {
            double acc = 0.0;
            for (int d = 0; d < K; ++d)
                acc += qt[d] * S[(size_t)d * V + c];
            ot[c] = J->scale * acc;
        }
    }

    if (hs)
        memcpy(hs, S, sizeof(double) * (size_t)K * V);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const long nchains = (long)J->N * J->HV;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->K * J->V);
    double *p = (double *)malloc(sizeof(double) * (size_t)J->V);
    double *delta = (double *)malloc(sizeof(double) * (size_t)J->V);
    if (!S || !p || !delta) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
        free(S); free(p); free(delta);
        return NULL;
    }
    for (;;) {
        long c;
        pthread_mutex_lock(&J->lock);
        c = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (c >= nchains)
            break;
        run_chain(J, c, S, p, delta);
    }
    free(S); free(p); free(delta);
    return NULL;
}

/*
 * Returns 0 on success, KDA_ORACLE_BAD_CU_SEQLENS when cu_seqlens breaks
 * 0 = cu[0] <= cu[1] <= ... <= cu[N] <= T (nothing is written then), and
 * KDA_ORACLE_BAD_ARGS for inconsistent sizes.
 */
int kda_oracle_recurrent(const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *h0,
                         const int32_t *cu_seqlens, int N, double *o, double *ht,
                         int B, int T, int H, int HV, int K, int V, double scale,
                         int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0)
        return KDA_ORACLE_BAD_ARGS;
    if (cu_seqlens) {
        if (B != 1 || N < 0)
            return KDA_ORACLE_BAD_ARGS;
        if (cu_seqlens[0] != 0)
            return KDA_ORACLE_BAD_CU_SEQLENS;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n] < 0 || cu_seqlens[n] > cu_seqlens[n + 1] || cu_seqlens[n + 1] > T)
                return KDA_ORACLE_BAD_CU_SEQLENS;
    } else {
        N = B;
    }
    if (nthreads < 1)
        nthreads = 1;

    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.cu = cu_seqlens; J.o = o; J.ht = ht;
    J.B = B; J.T = T; J.H = H; J.HV = HV; J.K = K; J.V = V; J.N = N;
    J.scale = scale;
    J.next = 0;
    J.failed = 0;
    pthread_mutex_init(&J.lock, NULL);

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
        pthread_mutex_destroy(&J.lock);
        return KDA_ORACLE_NO_MEMORY;
    }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? KDA_ORACLE_NO_MEMORY : KDA_ORACLE_OK;
}
