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
    const double *erase, *write;  /* Gated DeltaNet-2 gates, or NULL for KDA */
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

/*
 * Gated DeltaNet-2, one unit, token by token ("线性注意力机制：从标准注意力到
 * Gated DeltaNet-2", jindou-blog, section 4 "Gated DeltaNet-2：解耦擦除与写入",
 * and its table of erase/write control).  The page splits the one scalar gate
 * of the delta rule, which scales both the removal of the old association and
 * the writing of the new one, into an erase gate e_t and a write gate w_t,
 * each a vector over the d channels.  Its printed update is garbled; the
 * reading taken here keeps KDA's steps (so that KDA, Gated DeltaNet and
 * linear attention are special cases, as the page's table claims) and gates
 * the two halves of the write per key channel (row i of S):
 *
 *   1. forget   S <- Diag(alpha_t) S
 *   2. predict  vhat = S^T k_t
 *   3. erase    S <- S - (e_t . k_t) vhat^T      ((e_t . k_t)_i = e_t[i] k_t[i])
 *   4. write    S <- S + (w_t . k_t) v_t^T
 *   5. read     o_t = scale * S^T q_t
 *
 * With e_t = w_t = beta_t 1 this is the KDA token step above; with e_t = 0 it
 * is a gated linear attention with a per-channel write gate.
 */
static void run_unit_gdn2(const job_t *J, long u, double *S, double *vhat)
{
    const int dk = J->dk, dv = J->dv;
    const long T = J->T;
    const double *q = J->q + u * T * dk;
    const double *k = J->k + u * T * dk;
    const double *a = J->alpha + u * T * dk;
    const double *er = J->erase + u * T * dk;
    const double *wr = J->write + u * T * dk;
    const double *v = J->v + u * T * dv;
    double *o = J->o ? J->o + u * T * dv : NULL;

    if (J->s0)
        memcpy(S, J->s0 + u * (long)dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (long t = 0; t < T; ++t) {
        const double *at = a + t * dk, *kt = k + t * dk, *qt = q + t * dk;
        const double *et = er + t * dk, *wt = wr + t * dk;
        const double *vt = v + t * dv;
        /* 1. forget */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] *= at[i];
        /* 2. predict */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[i * dv + j] * kt[i];
            vhat[j] = acc;
        }
        /* 3. erase and 4. write */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] += -et[i] * kt[i] * vhat[j] + wt[i] * kt[i] * vt[j];
        /* 5. read */
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
        if (J->erase)
            run_unit_gdn2(J, u, S, vhat);
        else
            run_unit(J, u, S, vhat);
    }
    free(S);
    free(vhat);
    return NULL;
}

static int run_job(job_t *Jp, int n_threads);

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
    J.erase = NULL; J.write = NULL;
    J.o = o; J.sT = sT;
    J.n_units = n_units; J.T = T; J.dk = dk; J.dv = dv; J.scale = scale;
    J.next_unit = 0;
    return run_job(&J, n_threads);
}

/* Runs J's units on n_threads threads (<= 0: one per online CPU). */
static int run_job(job_t *Jp, int n_threads)
{
    job_t J = *Jp;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads <= 0) {
        long nc = sysconf(_SC_NPROCESSORS_ONLN);
        n_threads = nc > 0 ? (int)nc : 1;
    }
    if (n_threads > J.n_units)
        n_threads = (int)J.n_units;

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

/*
 * Gradients of the token loop above, by the chain rule through its four steps
 * taken in reverse token order.  For one unit, with e_t = beta_t (v_t - vhat_t)
 * the written error and dS the gradient of the loss with respect to the state
 * after token t (dS_T given, zero if absent):
 *
 *   read      o_t = scale S_t^T q_t      dq_t  = scale S_t do_t
 *                                        dS   += scale q_t do_t^T
 *   write     S_t = S~ + k_t e_t^T       dk_t  = dS e_t,   de = dS^T k_t
 *   correct   e_t = beta_t (v_t - vhat)  dbeta_t = de . (v_t - vhat)
 *                                        dv_t  = beta_t de,  dvhat = -beta_t de
 *   predict   vhat = S~^T k_t            dS~   = dS + k_t dvhat^T
 *                                        dk_t += S~ dvhat
 *   forget    S~ = Diag(alpha_t) S_{t-1} dalpha_t[i] = sum_j dS~[i][j] S_{t-1}[i][j]
 *                                        dS    = Diag(alpha_t) dS~
 *
 * and dS_0 is dS after token 0.  The steps and their order are those of the
 * forward ("Kimi Delta Attention", section "KDA 的更新式"; bugfactory.tech
 * news 3610, second to fourth paragraphs).  The forward states S_{t-1} of the
 * unit are kept for the reverse sweep (T * dk * dv doubles per thread), so
 * nothing is recomputed and nothing is blocked.
 *
 * Layouts as for kda_oracle_forward; dout [n_units][T][dv]; dsT [n_units][dk][dv]
 * or NULL; the gradients have the shapes of their inputs (dbeta [n_units][T],
 * ds0 [n_units][dk][dv]).
 */
typedef struct {
    const double *q, *k, *v, *alpha, *beta, *s0, *dout, *dsT;
    double *gq, *gk, *gv, *ga, *gb, *gs0;
    long n_units, T;
    int dk, dv;
    double scale;
    long next_unit;
    pthread_mutex_t lock;
} bwd_job_t;

typedef struct {
    double *sprev;  /* [T][dk][dv]: S_{t-1} for every token */
    double *resid;  /* [T][dv]: v_t - vhat_t */
    double *S, *dS, *dSt, *vhat, *de;
} bwd_scratch_t;

static void bwd_unit(const bwd_job_t *J, long u, bwd_scratch_t *W)
{
    const int dk = J->dk, dv = J->dv;
    const long T = J->T, dd = (long)dk * dv;
    const double *q = J->q + u * T * dk, *k = J->k + u * T * dk;
    const double *a = J->alpha + u * T * dk, *b = J->beta + u * T;
    const double *v = J->v + u * T * dv, *dout = J->dout + u * T * dv;
    double *gq = J->gq + u * T * dk, *gk = J->gk + u * T * dk;
    double *gv = J->gv + u * T * dv, *ga = J->ga + u * T * dk, *gb = J->gb + u * T;
    double *S = W->S, *dS = W->dS, *dSt = W->dSt, *vhat = W->vhat, *de = W->de;

    /* forward sweep, keeping S_{t-1} and the residual v_t - vhat_t */
    if (J->s0)
        memcpy(S, J->s0 + u * dd, sizeof(double) * dd);
    else
        memset(S, 0, sizeof(double) * dd);
    for (long t = 0; t < T; ++t) {
        const double *at = a + t * dk, *kt = k + t * dk, *vt = v + t * dv;
        double *rt = W->resid + t * dv;
        memcpy(W->sprev + t * dd, S, sizeof(double) * dd);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] *= at[i];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[i * dv + j] * kt[i];
            rt[j] = vt[j] - acc;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] += b[t] * kt[i] * rt[j];
    }

    /* reverse sweep */
    if (J->dsT)
        memcpy(dS, J->dsT + u * dd, sizeof(double) * dd);
    else
        memset(dS, 0, sizeof(double) * dd);
    for (long t = T - 1; t >= 0; --t) {
        const double *at = a + t * dk, *kt = k + t * dk, *qt = q + t * dk;
        const double *dot = dout + t * dv, *rt = W->resid + t * dv;
        const double *sp = W->sprev + t * dd;
        const double bt = b[t];
        /* S~ = Diag(alpha_t) S_{t-1} (kept in dSt for now) and S_t = S~ + k e^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] = at[i] * sp[i * dv + j] + kt[i] * bt * rt[j];
        /* read */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j)
                acc += S[i * dv + j] * dot[j];
            gq[t * dk + i] = J->scale * acc;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                dS[i * dv + j] += J->scale * qt[i] * dot[j];
        /* write */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j)
                acc += dS[i * dv + j] * bt * rt[j];
            gk[t * dk + i] = acc;
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += dS[i * dv + j] * kt[i];
            de[j] = acc;
        }
        /* correct */
        {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j)
                acc += de[j] * rt[j];
            gb[t] = acc;
        }
        for (int j = 0; j < dv; ++j) {
            gv[t * dv + j] = bt * de[j];
            vhat[j] = -bt * de[j];  /* dvhat */
        }
        /* predict: dS~ = dS + k dvhat^T, dk += S~ dvhat */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                dSt[i * dv + j] = dS[i * dv + j] + kt[i] * vhat[j];
                acc += at[i] * sp[i * dv + j] * vhat[j];
            }
            gk[t * dk + i] += acc;
        }
        /* forget */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j)
                acc += dSt[i * dv + j] * sp[i * dv + j];
            ga[t * dk + i] = acc;
            for (int j = 0; j < dv; ++j)
                dS[i * dv + j] = at[i] * dSt[i * dv + j];
        }
    }
    memcpy(J->gs0 + u * dd, dS, sizeof(double) * dd);
}

static void *bwd_worker(void *arg)
{
    bwd_job_t *J = (bwd_job_t *)arg;
    const long dd = (long)J->dk * J->dv;
    bwd_scratch_t W;
    W.sprev = (double *)malloc(sizeof(double) * (J->T > 0 ? J->T : 1) * dd);
    W.resid = (double *)malloc(sizeof(double) * (J->T > 0 ? J->T : 1) * J->dv);
    W.S = (double *)malloc(sizeof(double) * dd);
    W.dS = (double *)malloc(sizeof(double) * dd);
    W.dSt = (double *)malloc(sizeof(double) * dd);
    W.vhat = (double *)malloc(sizeof(double) * J->dv);
    W.de = (double *)malloc(sizeof(double) * J->dv);
    void *ret = NULL;
    if (!W.sprev || !W.resid || !W.S || !W.dS || !W.dSt || !W.vhat || !W.de) {
        ret = (void *)1;
    } else {
        for (;;) {
            pthread_mutex_lock(&J->lock);
            long u = J->next_unit++;
            pthread_mutex_unlock(&J->lock);
            if (u >= J->n_units)
                break;
            bwd_unit(J, u, &W);
        }
    }
    free(W.sprev); free(W.resid); free(W.S); free(W.dS); free(W.dSt);
    free(W.vhat); free(W.de);
    return ret;
}

/*
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 * n_threads <= 0 means one thread per online CPU.
 */
int kda_oracle_backward(const double *q, const double *k, const double *v,
                        const double *alpha, const double *beta, const double *s0,
                        const double *dout, const double *dsT,
                        double *gq, double *gk, double *gv, double *ga, double *gb,
                        double *gs0, long n_units, long T, int dk, int dv,
                        double scale, int n_threads)
{
    if (n_units < 0 || T < 0 || dk <= 0 || dv <= 0 || !gs0)
        return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !dout || !gq || !gk || !gv ||
                  !ga || !gb))
        return -1;
    if (n_units == 0)
        return 0;

    bwd_job_t J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.s0 = s0;
    J.dout = dout; J.dsT = dsT;
    J.gq = gq; J.gk = gk; J.gv = gv; J.ga = ga; J.gb = gb; J.gs0 = gs0;
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
        if (pthread_create(&tid[i], NULL, bwd_worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0 && bwd_worker(&J) != NULL)
        rc = -2;
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
 * Gated DeltaNet-2 forward (run_unit_gdn2) over n_units units: layouts as for
 * kda_oracle_forward with erase and write [n_units][T][dk] in place of beta.
 */
int gdn2_oracle_forward(const double *q, const double *k, const double *v,
                        const double *alpha, const double *erase, const double *write,
                        const double *s0, double *o, double *sT, long n_units, long T,
                        int dk, int dv, double scale, int n_threads)
{
    if (n_units < 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !erase || !write))
        return -1;
    if (n_units == 0)
        return 0;
    job_t J;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = NULL; J.s0 = s0;
    J.erase = erase ? erase : q;  /* T == 0: any non-NULL marks the mode */
    J.write = write;
    J.o = o; J.sT = sT;
    J.n_units = n_units; J.T = T; J.dk = dk; J.dv = dv; J.scale = scale;
    J.next_unit = 0;
    return run_job(&J, n_threads);
}

