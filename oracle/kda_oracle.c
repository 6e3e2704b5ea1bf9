/*
 * kda_oracle.c -- plain, slow, token-serial FP64 oracle for the KDA core.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code with the HIP library.
 *
 * What it computes (one independent unit per (sequence, head)):
 *
 *   Ling-3.1-flash: Grouped Routing and Two Different MLA Caches (flozi.net),
 *   section "KDA replaces a token list with a recurrent matrix": each head keeps
 *   a recurrent matrix; per token the kernel applies channel-dependent retention,
 *   then a delta-rule write that corrects the state's prediction for the current
 *   key toward the current value, then reads the matrix with the query. The same
 *   section fixes the safe forget gate's log-retention lower bound at -5.
 *
 *   In symbols, with the state S of shape dk x dv (rows = key channels):
 *     S'  = Diag(exp(max(g_t, lb))) S_{t-1}       retention, per key channel
 *     u   = beta_t (v_t - S'^T k_t)                 corrected write
 *     S_t = S' + k_t u^T                            = (I - b k k^T) Diag(a) S + b k v^T
 *     o_t = scale * S_t^T q_t                       read after the write
 *
 *   The update with an uncorrected k v^T term printed on the page
 *   "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its safetensors
 *   headers" (section "How KDA and MLA split the work", the displayed equation)
 *   lacks the correction term that the flozi.net page describes in words; the
 *   delta form is the reading taken here.
 *
 * Precision: inputs are float32 arrays (bf16 inputs are exactly representable);
 * every operation is done in double. No blocking, no reordering of the
 * recurrence: tokens are visited strictly in order.
 *
 * Build: gcc -O2 -shared -fPIC -o liboracle.so kda_oracle.c -lm -lpthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *g, *beta;
    int64_t total_tokens;
    int H, dk, dv;
    const int64_t *cu_seqlens;
    int num_seqs;
    double scale, lower_bound;
    const double *s0; /* [N,H,dk,dv] or NULL */
    double *o;        /* [T,H,dv] */
    double *sT;       /* [N,H,dk,dv] or NULL */
    int64_t next_unit;
    pthread_mutex_t lock;
    int failed;
} job_t;

/* One (sequence, head) unit, token by token. */
static int run_unit(job_t *J, int n, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *a = (double *)malloc(sizeof(double) * (size_t)dk);
    if (!S || !p || !a) {
        free(S); free(p); free(a);
        return -1;
    }
    const size_t sbase = ((size_t)n * H + h) * (size_t)dk * dv;
    if (J->s0)
        memcpy(S, J->s0 + sbase, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);

    for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
        const float *qt = J->q + ((size_t)t * H + h) * dk;
        const float *kt = J->k + ((size_t)t * H + h) * dk;
        const float *gt = J->g + ((size_t)t * H + h) * dk;
        const float *vt = J->v + ((size_t)t * H + h) * dv;
        const double bt = (double)J->beta[(size_t)t * H + h];
        double *ot = J->o + ((size_t)t * H + h) * dv;

        /* retention: scale row c (key channel c) by alpha_c = exp(max(g_c, lb)) */
        for (int c = 0; c < dk; ++c) {
            double gc = (double)gt[c];
            if (gc < J->lower_bound) gc = J->lower_bound;
            a[c] = exp(gc);
        }
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j)
                S[(size_t)c * dv + j] *= a[c];

        /* prediction of the retained state for the current key: p = S'^T k */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            for (int j = 0; j < dv; ++j) p[j] += kc * S[(size_t)c * dv + j];
        }
        /* corrected write u = beta (v - p); S += k u^T */
        for (int j = 0; j < dv; ++j) p[j] = bt * ((double)vt[j] - p[j]);
        for (int c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kc * p[j];
        }
        /* read after the write: o = scale * S^T q */
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            const double qc = (double)qt[c];
            for (int j = 0; j < dv; ++j) ot[j] += qc * S[(size_t)c * dv + j];
        }
        for (int j = 0; j < dv; ++j) ot[j] *= J->scale;
    }
    if (J->sT) memcpy(J->sT + sbase, S, sizeof(double) * (size_t)dk * dv);
    free(S); free(p); free(a);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t units = (int64_t)J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        if (run_unit(J, (int)(u / J->H), (int)(u % J->H)) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/*
 * q,k,g : float32 [T, H, dk]      v : float32 [T, H, dv]      beta : float32 [T, H]
 * cu_seqlens : int64 [num_seqs+1], cu_seqlens[0] = 0, cu_seqlens[num_seqs] = T
 * s0 : double [num_seqs, H, dk, dv] or NULL (zero initial state)
 * o  : double [T, H, dv] (written)   sT : double [num_seqs, H, dk, dv] or NULL
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_kda_serial(const float *q, const float *k, const float *v, const float *g,
                      const float *beta, int64_t total_tokens, int H, int dk, int dv,
                      const int64_t *cu_seqlens, int num_seqs, double scale,
                      double lower_bound, const double *s0, double *o, double *sT,
                      int nthreads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return -1;
    if (H <= 0 || dk <= 0 || dv <= 0 || num_seqs <= 0 || total_tokens < 0) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != total_tokens) return -1;
    for (int n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.total_tokens = total_tokens; J.H = H; J.dk = dk; J.dv = dv;
    J.cu_seqlens = cu_seqlens; J.num_seqs = num_seqs;
    J.scale = scale; J.lower_bound = lower_bound;
    J.s0 = s0; J.o = o; J.sT = sT;
    pthread_mutex_init(&J.lock, NULL);

    const int64_t units = (int64_t)num_seqs * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    worker(&J); /* the calling thread works too */
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : 0;
}
