/*
 * kda_oracle_bwd.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The gradients of the token-by-token KDA recurrence (the forward in kda_oracle.c),
 * in fp64, by reverse-mode differentiation written out by hand, token by token. It
 * shares no code with the HIP library. Only the test suite and the benchmark's
 * CPU-baseline leg may load it.
 *
 * Forward, per sequence n and value head hv (q/k head h = hv / (HV/H)), token t:
 *     Sd  = Diag(2^g_t) S                 decay (S is the state before token t)
 *     p   = Sd^T k_t                      prediction
 *     del = beta_t (v_t - p)              correction
 *     S'  = Sd + k_t del^T                state after token t
 *     o_t = scale S'^T q_t
 * Given do (the gradient of a loss with respect to o) and dht (with respect to the
 * final state, or zeros), with A the gradient with respect to the current state S':
 *     dq_t     = scale S' do_t              A += scale q_t do_t^T
 *     dk_t     = A del                      ddel = A^T k_t
 *     dbeta_t  = ddel . (v_t - p)           dv_t = beta_t ddel       dp = -beta_t ddel
 *     dSd      = A + k_t dp^T               dk_t += Sd dp
 *     dg_t[d]  = ln 2 * sum_v dSd[d, v] Sd[d, v]     (g is the per-token log2 decay)
 *     A        = Diag(2^g_t) dSd            (the gradient with respect to S)
 * and the gradient with respect to the initial state is the final A. dq and dk of the
 * value heads that share a q/k head are summed. The forward is the one of the pages
 * ("kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md: intro and section Forward); its
 * backward ("Backward", same page) returns dq, dk, dv, dbeta, dg with respect to the
 * pre-cumsum decay and dh0, which is what this computes.
 *
 * The states of each chain are recomputed from checkpoints taken every SEG tokens of
 * the forward, so memory stays at one checkpoint per SEG tokens plus SEG states.
 *
 * Layouts as the forward oracle; do [B, T, HV, V], dht and dh0 [N, HV, K, V].
 * Outputs dq, dk [B, T, H, K], dv [B, T, HV, V], dg [B, T, HV, K], dbeta [B, T, HV];
 * rows outside every sequence get zeros. An empty sequence passes dht to dh0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SEG 64

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0, *dout, *dht;
    const int32_t *cu;
    double *dq_hv, *dk_hv, *dv, *dg, *dbeta, *dh0;
    int B, T, H, HV, K, V, N;
    double scale;
    long next;
    int failed;
    pthread_mutex_t lock;
} bjob_t;

typedef struct {
    double *ckpt;    /* [nseg][K*V] states at segment starts */
    double *states;  /* [SEG][K*V] states before each token of the current segment */
    double *S, *Sd, *A, *dSd, *p, *del, *ddel, *dp;
    long nseg_cap;
} work_t;

/* One forward token step on S (in place); p and del receive the prediction and the
 * correction. */
static void step(const double *qt, const double *kt, const double *vt, const double *gt,
                 double bt, double *S, double *p, double *del, int K, int V)
{
    (void)qt;
    for (int d = 0; d < K; ++d) {
        const double a = exp2(gt[d]);
        for (int c = 0; c < V; ++c)
            S[(size_t)d * V + c] *= a;
    }
    for (int c = 0; c < V; ++c)
        p[c] = 0.0;
    for (int d = 0; d < K; ++d)
        for (int c = 0; c < V; ++c)
            p[c] += kt[d] * S[(size_t)d * V + c];
    for (int c = 0; c < V; ++c)
        del[c] = bt * (vt[c] - p[c]);
    for (int d = 0; d < K; ++d)
        for (int c = 0; c < V; ++c)
            S[(size_t)d * V + c] += kt[d] * del[c];
}

static void run_chain(bjob_t *J, long chain, work_t *W)
{
    const int K = J->K, V = J->V, H = J->H, HV = J->HV, T = J->T;
    const size_t KV = (size_t)K * V;
    const int n = (int)(chain / HV);
    const int hv = (int)(chain % HV);
    const int h = hv / (HV / H);
    long row0, bos, eos;
    if (J->cu) {
        row0 = 0;
        bos = J->cu[n];
        eos = J->cu[n + 1];
    } else {
        row0 = (long)n * T;
        bos = 0;
        eos = T;
    }
    const size_t sofs = ((size_t)n * HV + hv) * KV;
    const long len = eos - bos;
    const long nseg = (len + SEG - 1) / SEG;
    double *S = W->S, *Sd = W->Sd, *A = W->A, *dSd = W->dSd;
    double *p = W->p, *del = W->del, *ddel = W->ddel, *dp = W->dp;
    const double LN2 = log(2.0);

    /* forward with checkpoints */
    if (J->h0)
        memcpy(S, J->h0 + sofs, sizeof(double) * KV);
    else
        memset(S, 0, sizeof(double) * KV);
    for (long t = bos; t < eos; ++t) {
        const long i = t - bos;
        if (i % SEG == 0)
            memcpy(W->ckpt + (size_t)(i / SEG) * KV, S, sizeof(double) * KV);
        const size_t r = (size_t)(row0 + t);
        step(J->q + (r * H + h) * K, J->k + (r * H + h) * K, J->v + (r * HV + hv) * V,
             J->g + (r * HV + hv) * K, J->beta[r * HV + hv], S, p, del, K, V);
    }

    /* backward */
    if (J->dht)
        memcpy(A, J->dht + sofs, sizeof(double) * KV);
    else
        memset(A, 0, sizeof(double) * KV);
    for (long sgi = nseg - 1; sgi >= 0; --sgi) {
        const long t0 = bos + sgi * SEG;
        const long t1 = t0 + SEG < eos ? t0 + SEG : eos;
        memcpy(S, W->ckpt + (size_t)sgi * KV, sizeof(double) * KV);
        for (long t = t0; t < t1; ++t) {
            memcpy(W->states + (size_t)(t - t0) * KV, S, sizeof(double) * KV);
            const size_t r = (size_t)(row0 + t);
            step(J->q + (r * H + h) * K, J->k + (r * H + h) * K, J->v + (r * HV + hv) * V,
                 J->g + (r * HV + hv) * K, J->beta[r * HV + hv], S, p, del, K, V);
        }
        for (long t = t1 - 1; t >= t0; --t) {
            const size_t r = (size_t)(row0 + t);
            const double *qt = J->q + (r * H + h) * K;
            const double *kt = J->k + (r * H + h) * K;
            const double *vt = J->v + (r * HV + hv) * V;
            const double *gt = J->g + (r * HV + hv) * K;
            const double bt = J->beta[r * HV + hv];
            const double *dot = J->dout + (r * HV + hv) * V;
            double *dqt = J->dq_hv + (r * HV + hv) * K;
            double *dkt = J->dk_hv + (r * HV + hv) * K;
            double *dvt = J->dv + (r * HV + hv) * V;
            double *dgt = J->dg + (r * HV + hv) * K;
            const double *Sprev = W->states + (size_t)(t - t0) * KV;

            /* recompute Sd, p, del and the state after the token */
            for (int d = 0; d < K; ++d) {
                const double a = exp2(gt[d]);
                for (int c = 0; c < V; ++c)
                    Sd[(size_t)d * V + c] = a * Sprev[(size_t)d * V + c];
            }
            for (int c = 0; c < V; ++c)
                p[c] = 0.0;
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c)
                    p[c] += kt[d] * Sd[(size_t)d * V + c];
            for (int c = 0; c < V; ++c)
                del[c] = bt * (vt[c] - p[c]);
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c)
                    S[(size_t)d * V + c] = Sd[(size_t)d * V + c] + kt[d] * del[c];

            /* o_t = scale S'^T q_t */
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c)
                    acc += S[(size_t)d * V + c] * dot[c];
                dqt[d] = J->scale * acc;
            }
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c)
                    A[(size_t)d * V + c] += J->scale * qt[d] * dot[c];
            /* S' = Sd + k del^T */
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c)
                    acc += A[(size_t)d * V + c] * del[c];
                dkt[d] = acc;
            }
            for (int c = 0; c < V; ++c) {
                double acc = 0.0;
                for (int d = 0; d < K; ++d)
                    acc += A[(size_t)d * V + c] * kt[d];
                ddel[c] = acc;
            }
            /* del = beta (v - p) */
            {
                double acc = 0.0;
                for (int c = 0; c < V; ++c)
                    acc += ddel[c] * (vt[c] - p[c]);
                J->dbeta[r * HV + hv] = acc;
            }
            for (int c = 0; c < V; ++c) {
                dvt[c] = bt * ddel[c];
                dp[c] = -bt * ddel[c];
            }
            /* p = Sd^T k */
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c)
                    dSd[(size_t)d * V + c] = A[(size_t)d * V + c] + kt[d] * dp[c];
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c)
                    acc += Sd[(size_t)d * V + c] * dp[c];
                dkt[d] += acc;
            }
            /* Sd = Diag(2^g) S */
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c)
                    acc += dSd[(size_t)d * V + c] * Sd[(size_t)d * V + c];
                dgt[d] = LN2 * acc;
            }
            for (int d = 0; d < K; ++d) {
                const double a = exp2(gt[d]);
                for (int c = 0; c < V; ++c)
                    A[(size_t)d * V + c] = a * dSd[(size_t)d * V + c];
            }
        }
    }
    if (J->dh0)
        memcpy(J->dh0 + sofs, A, sizeof(double) * KV);
}

static void *bworker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    const long nchains = (long)J->N * J->HV;
    const size_t KV = (size_t)J->K * J->V;
    long maxlen = J->T;
    work_t W;
    memset(&W, 0, sizeof(W));
    W.nseg_cap = (maxlen + SEG - 1) / SEG + 1;
    W.ckpt = (double *)malloc(sizeof(double) * KV * (size_t)W.nseg_cap);
    W.states = (double *)malloc(sizeof(double) * KV * SEG);
    W.S = (double *)malloc(sizeof(double) * KV);
    W.Sd = (double *)malloc(sizeof(double) * KV);
    W.A = (double *)malloc(sizeof(double) * KV);
    W.dSd = (double *)malloc(sizeof(double) * KV);
    W.p = (double *)malloc(sizeof(double) * (size_t)J->V);
    W.del = (double *)malloc(sizeof(double) * (size_t)J->V);
    W.ddel = (double *)malloc(sizeof(double) * (size_t)J->V);
    W.dp = (double *)malloc(sizeof(double) * (size_t)J->V);
    if (!W.ckpt || !W.states || !W.S || !W.Sd || !W.A || !W.dSd || !W.p || !W.del || !W.ddel || !W.dp) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
    } else {
        for (;;) {
            long c;
            pthread_mutex_lock(&J->lock);
            c = J->next++;
            pthread_mutex_unlock(&J->lock);
            if (c >= nchains)
                break;
            run_chain(J, c, &W);
        }
    }
    free(W.ckpt); free(W.states); free(W.S); free(W.Sd); free(W.A); free(W.dSd);
    free(W.p); free(W.del); free(W.ddel); free(W.dp);
    return NULL;
}

/*
 * Returns 0 on success, -2 for a malformed cu_seqlens, -1 for inconsistent sizes,
 * -3 when memory runs out. The caller zero-fills every output; dq_hv and dk_hv are
 * [B, T, HV, K] scratch arrays the per-value-head gradients are written to before the
 * sum over each q/k head's value heads lands in dq and dk.
 */
int kda_oracle_recurrent_bwd(const double *q, const double *k, const double *v,
                             const double *g, const double *beta, const double *h0,
                             const int32_t *cu_seqlens, int N, const double *dout,
                             const double *dht, double *dq, double *dk, double *dv,
                             double *dg, double *dbeta, double *dh0, double *dq_hv,
                             double *dk_hv, int B, int T, int H, int HV, int K, int V,
                             double scale, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0)
        return -1;
    if (cu_seqlens) {
        if (B != 1 || N < 0)
            return -1;
        if (cu_seqlens[0] != 0)
            return -2;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n] < 0 || cu_seqlens[n] > cu_seqlens[n + 1] || cu_seqlens[n + 1] > T)
                return -2;
    } else {
        N = B;
    }
    if (nthreads < 1)
        nthreads = 1;
    bjob_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.dout = dout; J.dht = dht;
    J.cu = cu_seqlens;
    J.dq_hv = dq_hv; J.dk_hv = dk_hv; J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
    J.B = B; J.T = T; J.H = H; J.HV = HV; J.K = K; J.V = V; J.N = N;
    J.scale = scale;
    J.next = 0;
    J.failed = 0;
    pthread_mutex_init(&J.lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
        pthread_mutex_destroy(&J.lock);
        return -3;
    }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bworker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0)
        bworker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    if (J.failed)
        return -3;
    /* dq, dk of a q/k head: the sum over the value heads that read it */
    const int G = HV / H;
    for (long r = 0; r < (long)B * T; ++r)
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < K; ++d) {
                double sq = 0.0, sk = 0.0;
                for (int j = 0; j < G; ++j) {
                    sq += dq_hv[((size_t)r * HV + h * G + j) * K + d];
                    sk += dk_hv[((size_t)r * HV + h * G + j) * K + d];
                }
                dq[((size_t)r * H + h) * K + d] = sq;
                dk[((size_t)r * H + h) * K + d] = sk;
            }
    return 0;
}
