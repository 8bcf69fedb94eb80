/*
 * gdn2_oracle.c -- plain, slow, fp64 CPU reference of the Gated DeltaNet-2
 * (GDN-2) recurrence.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by the smoke check and by the CPU-baseline leg of the benchmark, never by
 * the library's product path.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (page "Why NVIDIA Gated DeltaNet-2 separates erase and
 * write gates", axbrief.com, section "Gated Delta Rule-2: channel-wise
 * separation of erase and write", the recurrence equation):
 *
 *     S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *
 * with S in R^{dk x dv} (rows = key channels), a per-key-channel decay
 * alpha_t = exp(g_t) (g_t = log alpha_t, the input), an erase gate
 * b_t in [0,1]^dk and a write gate w_t in [0,1]^dv.  The same section reads
 * the update as an online gradient step: decay the state, read it with the
 * gated key, and write the gated residual along k_t.  This file uses exactly
 * that residual (delta) form, which is algebraically identical to the
 * equation:
 *
 *     S'  = Diag(alpha_t) S_{t-1}
 *     r   = S'^T (b_t . k_t)
 *     u   = w_t . v_t - r
 *     S_t = S' + k_t u^T
 *     o_t = S_t^T q_t                  (read-out after the update)
 *
 * Readings where the pages are silent: read-out after the update; no 1/sqrt(dk)
 * query scale; the state orientation is dk x dv row-major.
 *
 * Layouts (all contiguous, row-major, double):
 *   q, k, b, log_alpha : [B, T, H, dk]     v, w, o : [B, T, H, dv]
 *   state              : [B, H, dk, dv]
 * Independent (b, h) sequences are spread over a small pthread pool.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

typedef struct {
    const double *q, *k, *v, *g, *b, *w, *s0;
    double *o, *s_final;
    int64_t B, T, H, dk, dv;
    /* backward only */
    const double *d_o, *d_sT;
    double *dq, *dk_, *dv_, *dg, *db, *dw, *ds0;
    int64_t next_task; /* guarded by lock */
    pthread_mutex_t lock;
    int err;
} job_t;

static int64_t take_task(job_t* j) {
    pthread_mutex_lock(&j->lock);
    int64_t t = j->next_task++;
    pthread_mutex_unlock(&j->lock);
    return t;
}

/* One step of the recurrence in residual form, on one (b,h) state.
 * tok_* point at the token's dk / dv vectors; scratch r, u have dv entries. */
static void step(double* S, int64_t dk, int64_t dv, const double* q, const double* k,
                 const double* v, const double* g, const double* b, const double* w,
                 double* o, double* r, double* u) {
    /* decay the rows (key channels) */
    for (int64_t c = 0; c < dk; ++c) {
        double a = exp(g[c]);
        double* row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) row[j] *= a;
    }
    /* gated read of the decayed state */
    for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        double bk = b[c] * k[c];
        const double* row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) r[j] += row[j] * bk;
    }
    /* gated residual, then write along k */
    for (int64_t j = 0; j < dv; ++j) u[j] = w[j] * v[j] - r[j];
    for (int64_t c = 0; c < dk; ++c) {
        double* row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) row[j] += k[c] * u[j];
    }
    /* read-out after the update */
    if (o) {
        for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double* row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) o[j] += row[j] * q[c];
        }
    }
}

static void* fwd_worker(void* arg) {
    job_t* j = (job_t*)arg;
    const int64_t dk = j->dk, dv = j->dv, H = j->H, T = j->T;
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !r || !u) {
        pthread_mutex_lock(&j->lock);
        j->err = ORACLE_ENOMEM;
        pthread_mutex_unlock(&j->lock);
        free(S); free(r); free(u);
        return NULL;
    }
    for (;;) {
        int64_t task = take_task(j);
        if (task >= j->B * H) break;
        int64_t bi = task / H, h = task % H;
        if (j->s0) memcpy(S, j->s0 + task * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (int64_t t = 0; t < T; ++t) {
            int64_t tk = ((bi * T + t) * H + h) * dk;
            int64_t tv = ((bi * T + t) * H + h) * dv;
            step(S, dk, dv, j->q + tk, j->k + tk, j->v + tv, j->g + tk, j->b + tk, j->w + tv,
                 j->o + tv, r, u);
        }
        if (j->s_final) memcpy(j->s_final + task * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    }
    free(S); free(r); free(u);
    return NULL;
}

static int run_pool(job_t* j, int nthreads, void* (*fn)(void*)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    j->next_task = 0;
    j->err = ORACLE_OK;
    pthread_mutex_init(&j->lock, NULL);
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[started], NULL, fn, j) == 0) ++started;
    }
    fn(j);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&j->lock);
    return j->err;
}

/* Forward over a whole sequence batch.  s0 may be NULL (zero initial state);
 * s_final may be NULL.  Returns 0 on success. */
int gdn2_oracle_fwd(const double* q, const double* k, const double* v, const double* log_alpha,
                    const double* b, const double* w, const double* s0, double* o,
                    double* s_final, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                    int nthreads) {
    if (!q || !k || !v || !log_alpha || !b || !w || !o) return ORACLE_EINVAL;
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return ORACLE_EINVAL;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.q = q; j.k = k; j.v = v; j.g = log_alpha; j.b = b; j.w = w; j.s0 = s0;
    j.o = o; j.s_final = s_final;
    j.B = B; j.T = T; j.H = H; j.dk = dk; j.dv = dv;
    return run_pool(&j, nthreads, fwd_worker);
}

/* One recurrent decode step for N independent sequences: exactly one
 * iteration of the forward's time loop.  state [N,H,dk,dv] is updated in
 * place; o [N,H,dv]. */
int gdn2_oracle_decode(const double* q, const double* k, const double* v, const double* log_alpha,
                       const double* b, const double* w, double* state, double* o, int64_t N,
                       int64_t H, int64_t dk, int64_t dv, int nthreads) {
    if (!state) return ORACLE_EINVAL;
    /* A decode step is the forward with T = 1, the state both read and written. */
    return gdn2_oracle_fwd(q, k, v, log_alpha, b, w, state, o, state, N, 1, H, dk, dv, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Vector-Jacobian product (reverse sweep) of the forward above.
 *
 * The same page notes that the backward pass cannot reuse the scalar shortcut
 * of the single-gate rule, because the two channel gates sit inside the
 * gradient-accumulating inner products; the gradient is taken here step by
 * step through the residual form, which carries those gates explicitly.
 * For a loss L = sum(d_o . o) + sum(d_sT . S_T), per step in reverse, with G
 * the gradient with respect to S_t:
 *
 *   G  += q_t d_o_t^T            dq_t  = S_t d_o_t
 *   dk_t += G u                  du    = G^T k_t
 *   dw_t = du . v_t              dv_t  = du . w_t        dr = -du
 *   dS'  = G + khat dr^T         dkhat = S' dr           (khat = b_t . k_t)
 *   db_t = dkhat . k_t           dk_t += dkhat . b_t
 *   dg_t[c] = sum_j dS'[c,j] S'[c,j]                     (d/d log alpha)
 *   G    = Diag(alpha_t) dS'     (gradient with respect to S_{t-1})
 *
 * States are recomputed forward from checkpoints taken every CKPT steps. */
#define CKPT 64

static void* vjp_worker(void* arg) {
    job_t* j = (job_t*)arg;
    const int64_t dk = j->dk, dv = j->dv, H = j->H, T = j->T;
    const int64_t n_ck = (T + CKPT - 1) / CKPT;
    const size_t ss = (size_t)(dk * dv);
    /* checkpoints: state entering step c*CKPT; segment: states after each step */
    double* ck = (double*)malloc(sizeof(double) * ss * (size_t)(n_ck > 0 ? n_ck : 1));
    double* seg = (double*)malloc(sizeof(double) * ss * (CKPT + 1));
    double* G = (double*)malloc(sizeof(double) * ss);
    double* dSp = (double*)malloc(sizeof(double) * ss);
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dkh = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!ck || !seg || !G || !dSp || !r || !u || !du || !dkh) {
        pthread_mutex_lock(&j->lock);
        j->err = ORACLE_ENOMEM;
        pthread_mutex_unlock(&j->lock);
        goto done;
    }
    for (;;) {
        int64_t task = take_task(j);
        if (task >= j->B * H) break;
        int64_t bi = task / H, h = task % H;
        double* S = seg; /* running state */
        if (j->s0) memcpy(S, j->s0 + task * ss, sizeof(double) * ss);
        else memset(S, 0, sizeof(double) * ss);
        /* forward pass recording checkpoints */
        for (int64_t t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (t / CKPT) * ss, S, sizeof(double) * ss);
            int64_t tk = ((bi * T + t) * H + h) * dk;
            int64_t tv = ((bi * T + t) * H + h) * dv;
            step(S, dk, dv, j->q + tk, j->k + tk, j->v + tv, j->g + tk, j->b + tk, j->w + tv,
                 NULL, r, u);
        }
        if (j->d_sT) memcpy(G, j->d_sT + task * ss, sizeof(double) * ss);
        else memset(G, 0, sizeof(double) * ss);
        for (int64_t c0 = n_ck - 1; c0 >= 0; --c0) {
            int64_t t0 = c0 * CKPT;
            int64_t t1 = t0 + CKPT < T ? t0 + CKPT : T;
            /* seg[i] = state entering step t0+i, i = 0..t1-t0 */
            memcpy(seg, ck + c0 * ss, sizeof(double) * ss);
            for (int64_t t = t0; t < t1; ++t) {
                double* nxt = seg + (t - t0 + 1) * ss;
                memcpy(nxt, seg + (t - t0) * ss, sizeof(double) * ss);
                int64_t tk = ((bi * T + t) * H + h) * dk;
                int64_t tv = ((bi * T + t) * H + h) * dv;
                step(nxt, dk, dv, j->q + tk, j->k + tk, j->v + tv, j->g + tk, j->b + tk,
                     j->w + tv, NULL, r, u);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                int64_t tk = ((bi * T + t) * H + h) * dk;
                int64_t tv = ((bi * T + t) * H + h) * dv;
                const double *q = j->q + tk, *k = j->k + tk, *v = j->v + tv, *g = j->g + tk;
                const double *b = j->b + tk, *w = j->w + tv, *dO = j->d_o + tv;
                const double* Sprev = seg + (t - t0) * ss;
                const double* Scur = seg + (t - t0 + 1) * ss;
                double *dq = j->dq + tk, *dkk = j->dk_ + tk, *dvv = j->dv_ + tv;
                double *dg = j->dg + tk, *db = j->db + tk, *dw = j->dw + tv;
                /* o_t = S_t^T q_t */
                for (int64_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int64_t jj = 0; jj < dv; ++jj) {
                        G[c * dv + jj] += q[c] * dO[jj];
                        acc += Scur[c * dv + jj] * dO[jj];
                    }
                    dq[c] = acc;
                }
                /* recompute S' and u of this step */
                for (int64_t jj = 0; jj < dv; ++jj) r[jj] = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    double a = exp(g[c]);
                    for (int64_t jj = 0; jj < dv; ++jj)
                        r[jj] += a * Sprev[c * dv + jj] * (b[c] * k[c]);
                }
                for (int64_t jj = 0; jj < dv; ++jj) u[jj] = w[jj] * v[jj] - r[jj];
                /* S_t = S' + k u^T */
                for (int64_t jj = 0; jj < dv; ++jj) du[jj] = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int64_t jj = 0; jj < dv; ++jj) {
                        acc += G[c * dv + jj] * u[jj];
                        du[jj] += G[c * dv + jj] * k[c];
                    }
                    dkk[c] = acc;
                }
                /* u = w.v - r */
                for (int64_t jj = 0; jj < dv; ++jj) {
                    dw[jj] = du[jj] * v[jj];
                    dvv[jj] = du[jj] * w[jj];
                }
                /* r = S'^T khat, dr = -du */
                for (int64_t c = 0; c < dk; ++c) {
                    double a = exp(g[c]);
                    double kh = b[c] * k[c];
                    double acc_dkh = 0.0, acc_dg = 0.0;
                    for (int64_t jj = 0; jj < dv; ++jj) {
                        double sp = a * Sprev[c * dv + jj];
                        double dsp = G[c * dv + jj] - kh * du[jj];
                        dSp[c * dv + jj] = dsp;
                        acc_dkh += -sp * du[jj];
                        acc_dg += dsp * sp;
                    }
                    dkh[c] = acc_dkh;
                    dg[c] = acc_dg;
                    db[c] = acc_dkh * k[c];
                    dkk[c] += acc_dkh * b[c];
                    for (int64_t jj = 0; jj < dv; ++jj) G[c * dv + jj] = a * dSp[c * dv + jj];
                }
            }
        }
        if (j->ds0) memcpy(j->ds0 + task * ss, G, sizeof(double) * ss);
    }
done:
    free(ck); free(seg); free(G); free(dSp); free(r); free(u); free(du); free(dkh);
    return NULL;
}

/* Gradients of L = sum(d_o . o) + sum(d_sT . S_T) with respect to every
 * input.  d_sT and s0 may be NULL (zeros); ds0 may be NULL. */
int gdn2_oracle_vjp(const double* q, const double* k, const double* v, const double* log_alpha,
                    const double* b, const double* w, const double* s0, const double* d_o,
                    const double* d_sT, double* dq, double* dk, double* dv_, double* dlog_alpha,
                    double* db, double* dw, double* ds0, int64_t B, int64_t T, int64_t H,
                    int64_t dk_dim, int64_t dv_dim, int nthreads) {
    if (!q || !k || !v || !log_alpha || !b || !w || !d_o) return ORACLE_EINVAL;
    if (!dq || !dk || !dv_ || !dlog_alpha || !db || !dw) return ORACLE_EINVAL;
    if (B < 1 || T < 0 || H < 1 || dk_dim < 1 || dv_dim < 1) return ORACLE_EINVAL;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.q = q; j.k = k; j.v = v; j.g = log_alpha; j.b = b; j.w = w; j.s0 = s0;
    j.d_o = d_o; j.d_sT = d_sT;
    j.dq = dq; j.dk_ = dk; j.dv_ = dv_; j.dg = dlog_alpha; j.db = db; j.dw = dw; j.ds0 = ds0;
    j.B = B; j.T = T; j.H = H; j.dk = dk_dim; j.dv = dv_dim;
    return run_pool(&j, nthreads, vjp_worker);
}

const char* gdn2_oracle_version(void) { return "gdn2-oracle fp64 1"; }
