/*
 * fp64 CPU oracle for the gated delta rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (per batch b and head h, all in IEEE double, plain serial
 * loops, no BLAS, no reassociation):
 *
 *   A   = -exp(A_log[h])                       (a per-head scalar kept in log
 *                                                space, decay alpha in (0,1):
 *                                                "GDN & MLA Mechanism
 *                                                Deep-Dive", Intuition and
 *                                                Step 4)
 *   alpha_t = exp(g_t * A)
 *   delta on  (gated delta rule, "HyMo-434M documentation portal",
 *              FIG. A0 probe and 01 GDN RECURRENCE, with the erase key
 *              read as k_t):
 *       u   = h^T k_t
 *       h   = alpha_t (h - beta_t k_t u^T) + beta_t k_t v_t^T
 *   delta off (additive write, "GDN & MLA Mechanism Deep-Dive", Step 4
 *              write line, with write key b_t = beta_t k_t):
 *       h   = alpha_t h + beta_t k_t v_t^T
 *   read after write ("GDN & MLA Mechanism Deep-Dive", Step 4 read line):
 *       o_t = h^T q_t
 *
 * The state h is d_k x d_v, row-major (h[i*dv + j]).
 * Layouts: q,k [B,T,H,dk]; v,o [B,T,H,dv]; g,beta [B,T,H]; A_log [H];
 *          states [B,H,dk,dv].
 *
 * Backward: the manual reverse-mode derivative of the serial loop above
 * (chain rule step by step, states recomputed from checkpoints every 64
 * steps). Gradients are with respect to q,k,v,g,beta (post-sigmoid values as
 * passed in), A_log and h0; the upstream gradients are do and dhT.
 *
 * Step: one iteration of the forward loop from a carried state, written out
 * on its own.
 *
 * Threading: independent (b,h) units are spread over pthreads; each unit is
 * computed by exactly one thread in a fixed order, and the only cross-unit
 * sum (dA_log over b) is done afterwards in a fixed order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int B, T, H, dk, dv, delta;
    const double *q, *k, *v, *g, *beta, *A_log, *h0, *dout, *dhT;
    double *o, *hT;
    double *dq, *dkk, *dvv, *dg, *dbeta, *dA_part, *dh0;
    const int *units;
    int n_units;
    int next;               /* work counter, guarded by mu */
    int failed;
    pthread_mutex_t mu;
} job_t;

static size_t tok_idx(const job_t *J, int b, int t, int h) {
    return ((size_t)b * J->T + t) * J->H + h;
}

/* One forward step of the recurrence on state s (dk x dv), in place. */
static void step_state(int dk, int dv, int delta, double alpha, double beta,
                       const double *kt, const double *vt, double *s, double *u) {
    if (delta) {
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) u[j] += s[i * dv + j] * kt[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                s[i * dv + j] = alpha * (s[i * dv + j] - beta * kt[i] * u[j]) + beta * kt[i] * vt[j];
    } else {
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                s[i * dv + j] = alpha * s[i * dv + j] + beta * kt[i] * vt[j];
    }
}

static void read_state(int dk, int dv, const double *s, const double *qt, double *ot) {
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) ot[j] += s[i * dv + j] * qt[i];
}

static int take_unit(job_t *J) {
    pthread_mutex_lock(&J->mu);
    int n = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (n >= J->n_units) return -1;
    return J->units ? J->units[n] : n;
}

/* ---------------------------------------------------------------- forward */

static void fwd_unit(job_t *J, int unit) {
    const int b = unit / J->H, h = unit % J->H, dk = J->dk, dv = J->dv;
    const double A = -exp(J->A_log[h]);
    double *s = (double *)calloc((size_t)dk * dv, sizeof(double));
    double *u = (double *)calloc((size_t)dv, sizeof(double));
    if (!s || !u) { J->failed = 1; free(s); free(u); return; }
    if (J->h0) memcpy(s, J->h0 + (size_t)unit * dk * dv, sizeof(double) * dk * dv);
    for (int t = 0; t < J->T; ++t) {
        const size_t ti = tok_idx(J, b, t, h);
        const double alpha = exp(J->g[ti] * A);
        step_state(dk, dv, J->delta, alpha, J->beta[ti], J->k + ti * dk, J->v + ti * dv, s, u);
        read_state(dk, dv, s, J->q + ti * dk, J->o + ti * dv);
    }
    if (J->hT) memcpy(J->hT + (size_t)unit * dk * dv, s, sizeof(double) * dk * dv);
    free(s);
    free(u);
}

static void *fwd_worker(void *arg) {
    job_t *J = (job_t *)arg;
    for (int u; (u = take_unit(J)) >= 0;) fwd_unit(J, u);
    return NULL;
}

/* --------------------------------------------------------------- backward */

#define SEG 64

static void bwd_unit(job_t *J, int unit) {
    const int b = unit / J->H, h = unit % J->H, dk = J->dk, dv = J->dv, T = J->T;
    const size_t S = (size_t)dk * dv;
    const double A = -exp(J->A_log[h]);
    const int nseg = (T + SEG - 1) / SEG;
    double *ck = (double *)calloc((size_t)(nseg > 0 ? nseg : 1) * S, sizeof(double)); /* state before each segment */
    double *st = (double *)calloc((size_t)(SEG + 1) * S, sizeof(double)); /* states inside a segment */
    double *dh = (double *)calloc(S, sizeof(double));
    double *Hh = (double *)calloc(S, sizeof(double));
    double *u = (double *)calloc((size_t)dv, sizeof(double));
    double *Dk = (double *)calloc((size_t)dv, sizeof(double));
    double *Du = (double *)calloc((size_t)dk, sizeof(double));
    if (!ck || !st || !dh || !Hh || !u || !Dk || !Du) {
        J->failed = 1;
        goto out;
    }
    /* forward sweep: keep the state at the start of every segment */
    {
        double *s = st;
        if (J->h0) memcpy(s, J->h0 + (size_t)unit * S, sizeof(double) * S);
        for (int t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * S, s, sizeof(double) * S);
            const size_t ti = tok_idx(J, b, t, h);
            step_state(dk, dv, J->delta, exp(J->g[ti] * A), J->beta[ti], J->k + ti * dk, J->v + ti * dv, s, u);
        }
    }
    if (J->dhT) memcpy(dh, J->dhT + (size_t)unit * S, sizeof(double) * S);
    double acc_gdl = 0.0; /* sum over t of g_t * dlambda_t, lambda_t = g_t * A */
    for (int sg = nseg - 1; sg >= 0; --sg) {
        const int t0 = sg * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
        memcpy(st, ck + (size_t)sg * S, sizeof(double) * S);
        for (int t = t0; t < t1; ++t) {
            const size_t ti = tok_idx(J, b, t, h);
            memcpy(st + (size_t)(t - t0 + 1) * S, st + (size_t)(t - t0) * S, sizeof(double) * S);
            step_state(dk, dv, J->delta, exp(J->g[ti] * A), J->beta[ti], J->k + ti * dk, J->v + ti * dv,
                       st + (size_t)(t - t0 + 1) * S, u);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t ti = tok_idx(J, b, t, h);
            const double *hp = st + (size_t)(t - t0) * S;     /* h_{t-1} */
            const double *hn = st + (size_t)(t - t0 + 1) * S; /* h_t */
            const double *qt = J->q + ti * dk, *kt = J->k + ti * dk, *vt = J->v + ti * dv;
            const double *dot = J->dout + ti * dv;
            const double gt = J->g[ti], bt = J->beta[ti], alpha = exp(gt * A);
            double *dqt = J->dq + ti * dk, *dkt = J->dkk + ti * dk, *dvt = J->dvv + ti * dv;

            /* read o_t = h_t^T q_t */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dh[i * dv + j] += qt[i] * dot[j];
            for (int i = 0; i < dk; ++i) {
                double a = 0.0;
                for (int j = 0; j < dv; ++j) a += hn[i * dv + j] * dot[j];
                dqt[i] = a;
            }
            /* the pre-decay state that alpha multiplies */
            if (J->delta) {
                for (int j = 0; j < dv; ++j) u[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) u[j] += hp[i * dv + j] * kt[i];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) Hh[i * dv + j] = hp[i * dv + j] - bt * kt[i] * u[j];
            } else {
                memcpy(Hh, hp, sizeof(double) * S);
            }
            /* h_t = alpha * Hh + beta k v^T */
            double dalpha = 0.0;
            for (size_t e = 0; e < S; ++e) dalpha += dh[e] * Hh[e];
            const double dlam = alpha * dalpha; /* d/d lambda, alpha = exp(lambda) */
            J->dg[ti] = A * dlam;
            acc_gdl += gt * dlam;
            double db = 0.0;
            for (int i = 0; i < dk; ++i) {
                double a = 0.0;
                for (int j = 0; j < dv; ++j) a += dh[i * dv + j] * vt[j];
                dkt[i] = bt * a;
                db += kt[i] * a;
            }
            for (int j = 0; j < dv; ++j) dvt[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dvt[j] += dh[i * dv + j] * kt[i];
            for (int j = 0; j < dv; ++j) dvt[j] *= bt;
            /* D = alpha * dh is the gradient reaching Hh */
            for (size_t e = 0; e < S; ++e) dh[e] *= alpha;
            if (J->delta) {
                /* Hh = hp - beta k u^T, u = hp^T k */
                for (int j = 0; j < dv; ++j) Dk[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) Dk[j] += dh[i * dv + j] * kt[i]; /* D^T k */
                for (int i = 0; i < dk; ++i) {
                    double a = 0.0, c = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        a += dh[i * dv + j] * u[j];  /* (D u)_i */
                        c += hp[i * dv + j] * Dk[j]; /* (hp D^T k)_i */
                    }
                    Du[i] = a;
                    dkt[i] -= bt * (a + c);
                }
                for (int i = 0; i < dk; ++i) db -= kt[i] * Du[i];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) dh[i * dv + j] -= bt * kt[i] * Dk[j];
            }
            J->dbeta[ti] = db;
        }
    }
    if (J->dh0) memcpy(J->dh0 + (size_t)unit * S, dh, sizeof(double) * S);
    J->dA_part[unit] = A * acc_gdl; /* dA_log = dA/dA_log * sum g dlambda, dA/dA_log = A */
out:
    free(ck); free(st); free(dh); free(Hh); free(u); free(Dk); free(Du);
}

static void *bwd_worker(void *arg) {
    job_t *J = (job_t *)arg;
    for (int u; (u = take_unit(J)) >= 0;) bwd_unit(J, u);
    return NULL;
}

/* -------------------------------------------------------------- step */

static void step_unit(job_t *J, int unit) {
    /* here B plays the role of N (independent sequences), T == 1 */
    const int h = unit % J->H, dk = J->dk, dv = J->dv;
    const size_t S = (size_t)dk * dv, ti = (size_t)unit;
    const double A = -exp(J->A_log[h]);
    const double alpha = exp(J->g[ti] * A), bt = J->beta[ti];
    const double *kt = J->k + ti * dk, *vt = J->v + ti * dv, *qt = J->q + ti * dk;
    double *s = J->hT + (size_t)unit * S;
    if (J->h0) memcpy(s, J->h0 + (size_t)unit * S, sizeof(double) * S);
    else memset(s, 0, sizeof(double) * S);
    if (J->delta) {
        /* erase what k_t currently reads, decay, then write */
        for (int j = 0; j < dv; ++j) {
            double uj = 0.0;
            for (int i = 0; i < dk; ++i) uj += s[i * dv + j] * kt[i];
            for (int i = 0; i < dk; ++i)
                s[i * dv + j] = alpha * (s[i * dv + j] - bt * kt[i] * uj) + bt * kt[i] * vt[j];
        }
    } else {
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) s[i * dv + j] = alpha * s[i * dv + j] + bt * kt[i] * vt[j];
    }
    for (int j = 0; j < dv; ++j) {
        double a = 0.0;
        for (int i = 0; i < dk; ++i) a += s[i * dv + j] * qt[i];
        J->o[ti * dv + j] = a;
    }
}

static void *step_worker(void *arg) {
    job_t *J = (job_t *)arg;
    for (int u; (u = take_unit(J)) >= 0;) step_unit(J, u);
    return NULL;
}

/* ------------------------------------------------------- thread pool */

static int run(job_t *J, void *(*fn)(void *), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > J->n_units) nthreads = J->n_units > 0 ? J->n_units : 1;
    pthread_mutex_init(&J->mu, NULL);
    J->next = 0;
    J->failed = 0;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, fn, J) == 0) ++started;
    fn(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J->mu);
    return J->failed ? -2 : 0;
}

/* T = 0 is an empty sequence: no step of the recurrence runs, so the final
 * state is h0 and the gradient reaching h0 is dhT */
static int check_dims(int B, int T, int H, int dk, int dv) {
    return (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) ? -1 : 0;
}

/* units: optional list of b*H+h indices to compute (NULL = all B*H). Outputs
 * of units not listed are left untouched. */
int gdn_oracle_fwd(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                   const double *v, const double *g, const double *beta, const double *A_log,
                   const double *h0, int delta, double *o, double *hT, const int *units, int n_units,
                   int nthreads) {
    if (check_dims(B, T, H, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.delta = delta;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.A_log = A_log; J.h0 = h0;
    J.o = o; J.hT = hT;
    J.units = units;
    J.n_units = units ? n_units : B * H;
    return run(&J, fwd_worker, nthreads);
}

/* dA_log_part receives one entry per unit [B*H]; dA_log[h] = sum over b. */
int gdn_oracle_bwd(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                   const double *v, const double *g, const double *beta, const double *A_log,
                   const double *h0, const double *dout, const double *dhT, int delta, double *dq,
                   double *dk_out, double *dv_out, double *dg, double *dbeta, double *dA_log_part,
                   double *dh0, const int *units, int n_units, int nthreads) {
    if (check_dims(B, T, H, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.delta = delta;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.A_log = A_log; J.h0 = h0;
    J.dout = dout; J.dhT = dhT;
    J.dq = dq; J.dkk = dk_out; J.dvv = dv_out; J.dg = dg; J.dbeta = dbeta;
    J.dA_part = dA_log_part; J.dh0 = dh0;
    J.units = units;
    J.n_units = units ? n_units : B * H;
    return run(&J, bwd_worker, nthreads);
}

/* One token for each of N independent sequences: q,k [N,H,dk], v,o [N,H,dv],
 * g,beta [N,H], states [N,H,dk,dv]. h_in may be NULL (zero state). */
int gdn_oracle_step(int N, int H, int dk, int dv, const double *q, const double *k,
                    const double *v, const double *g, const double *beta, const double *A_log,
                    const double *h_in, int delta, double *o, double *h_out, int nthreads) {
    if (check_dims(N, 1, H, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = N; J.T = 1; J.H = H; J.dk = dk; J.dv = dv; J.delta = delta;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.A_log = A_log; J.h0 = h_in;
    J.o = o; J.hT = h_out;
    J.n_units = N * H;
    return run(&J, step_worker, nthreads);
}
