/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header or
 * constant with the HIP library; the product path never calls it.
 *
 * What it computes, per independent unit (one batch entry or sequence, one
 * head), with state S of shape dk x dv (row index = key channel, column index
 * = value channel), token by token in sequence order:
 *
 *   1. forget   S <- Diag(alpha_t) S
 *        "Kimi Delta Attention" (daiw.net, Kimi K3 manual), section
 *        "一、Diag(α_t)：通道级遗忘": alpha_t is a vector, one decay per key
 *        channel, applied to the old state.  bugfactory.tech news 3610,
 *        third paragraph (Gated DeltaNet): the state is decayed BEFORE the
 *        prediction; fourth paragraph (KDA): the scalar becomes a per-channel
 *        diagonal.
 *   2. predict  vhat = S^T k_t        (query the forgotten state with the key)
 *   3. correct  S <- S + beta_t k_t (v_t - vhat)^T   (write only the error)
 *        bugfactory.tech news 3610, second paragraph (DeltaNet: predict,
 *        error scaled by beta, write the error along the key);
 *        "Kimi Delta Attention", section "二、I − β_t k_t k_tᵀ：delta 规则".
 *        Steps 1-3 together are the update equation of section
 *        "KDA 的更新式":  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                              + beta_t k_t v_t^T.
 *   4. read     o_t = scale * S^T q_t, scale = dk^{-1/2} by default,
 *        with the state AFTER the write (bugfactory.tech news 3610, fourth
 *        paragraph: forget, predict, correct, write, then read with the
 *        dk^{-1/2} factor).
 *
 * Everything is double precision; inputs are the caller's stored values
 * already widened to double.  No blocking, no reordering, no fusion.
 *
 * Layout (all row-major, contiguous):
 *   q, k, alpha : [n_units][T][dk]
 *   v, o        : [n_units][T][dv]
 *   beta        : [n_units][T]
 *   s0, sT      : [n_units][dk][dv]   (s0 may be NULL = zero state)
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *alpha, *beta, *s0;
    double *o, *sT;
    long n_units, T;
    int dk, dv;
    double scale;
    long next_unit;          /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
} job_t;

/* One unit, token by token.  S and vhat are caller-provided scratch. */
static void run_unit(const job_t *J, long u, double *S, double *vhat)
{
    const int dk = J->dk, dv = J->dv;
    const long T = J->T;
    const double *q = J->q + u * T * dk;
    const double *k = J->k + u * T * dk;
    const double *a = J->alpha + u * T * dk;
    const double *v = J->v + u * T * dv;
    const double *b = J->beta + u * T;
    double *o = J->o ? J->o + u * T * dv : NULL;

    if (J->s0)
        memcpy(S, J->s0 + u * (long)dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (long t = 0; t < T; ++t) {
        const double *at = a + t * dk, *kt = k + t * dk, *qt = q + t * dk;
        const double *vt = v + t * dv;
        const double bt = b[t];

        /* 1. forget: row i of S is key channel i, scaled by alpha_t[i] */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] *= at[i];

        /* 2. predict: vhat = S^T k_t */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[i * dv + j] * kt[i];
            vhat[j] = acc;
        }

        /* 3. correct and write: S += beta_t k_t (v_t - vhat)^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] += bt * kt[i] * (vt[j] - vhat[j]);

        /* 4. read with the updated state: o_t = scale S^T q_t */
        if (o) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i)
                    acc += S[i * dv + j] * qt[i];
                o[t * dv + j] = J->scale * acc;
            }
        }
    }

    if (J->sT)
        memcpy(J->sT + u * (long)dk * dv, S, sizeof(double) * dk * dv);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * J->dk * J->dv);
    double *vhat = (double *)malloc(sizeof(double) * J->dv);
    if (!S || !vhat) {
        free(S);
        free(vhat);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        long u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= J->n_units)
            break;
        run_unit(J, u, S, vhat);
    }
    free(S);
    free(vhat);
    return NULL;
}

/*
 * Forward over n_units independent units of T tokens each.
 * o may be NULL (only the final state is wanted); sT may be NULL.
 * n_threads <= 0 means one thread per online CPU.
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *s0, double *o, double *sT,
                       long n_units, long T, int dk, int dv, double scale,
                       int n_threads)
{
    if (n_units < 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta))
        return -1;
    if (n_units == 0)
        return 0;

    job_t J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.s0 = s0;
    J.o = o; J.sT = sT;
    J.n_units = n_units; J.T = T; J.dk = dk; J.dv = dv; J.scale = scale;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads <= 0) {
        long nc = sysconf(_SC_NPROCESSORS_ONLN);
        n_threads = nc > 0 ? (int)nc : 1;
    }
    if (n_threads > n_units)
        n_threads = (int)n_units;

    int rc = 0;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * n_threads);
    if (!tid) {
        pthread_mutex_destroy(&J.lock);
        return -2;
    }
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0) {
        /* no thread could be started: run on the calling thread */
        if (worker(&J) != NULL)
            rc = -2;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret != NULL)
            rc = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return rc;
}

/*
 * One decode step for n_units units: exactly one iteration of the token loop
 * above per unit, reading and rewriting state [n_units][dk][dv] in place.
 * q, k, alpha: [n_units][dk]; v, o: [n_units][dv]; beta: [n_units].
 */
int kda_oracle_step(const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta, double *state,
                    double *o, long n_units, int dk, int dv, double scale,
                    int n_threads)
{
    if (!state)
        return -1;
    /* the forward reads s0 fully before writing sT for each unit, and units
     * are disjoint, so in-place use is safe */
    return kda_oracle_forward(q, k, v, alpha, beta, state, o, state,
                              n_units, 1, dk, dv, scale, n_threads);
}
