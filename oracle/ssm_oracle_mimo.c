/*
 * ssm_oracle_mimo.c -- plain fp64 CPU oracle for the multi-input
 * multi-output (MIMO) form of the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY, like ssm_oracle.c: nothing in the product
 * library links, loads or calls this file, and it shares no code with the
 * HIP path.
 *
 * What it computes.  Each (b, d) channel keeps ONE state vector h[n]
 * (n < N), as in the single-input scan, but every step brings R inputs
 * u[b,t,d,r] and produces R outputs y[b,t,d,r] (r < R).  B and C are N x R
 * per step instead of N-vectors:
 *
 *   q_t[n]   = sum_r Bm[b,t,n,r] * u[b,t,d,r]
 *   alpha, bterm and the state update are those of ssm_oracle.c with q_t in
 *   place of Bm[b,t,n] u[b,t,d]:
 *     z = delta A[d,n], alpha = e^z e^{i theta} (real state: e^z)
 *     ZOH   : bterm = expm1(z)/A q_t (delta q_t when A = 0)
 *     EULER : bterm = delta q_t
 *     TRAP  : bterm = lambda delta q_t + (1 - lambda) delta alpha q_{t-1}
 *     h[n]  = alpha h[n] + bterm
 *   y[b,t,d,r] = Re(sum_n Cm[b,t,n,r] h[n]) + Dskip[d] u[b,t,d,r]
 *
 * With R = 1 this is exactly the single-input scan.
 *
 * Sources (page title and section):
 *  - ai.tomabc.com Mamba-3 paper story, MIMO section and its shape table:
 *    B and C grow from N-vectors to N x P matrices (P parallel input/output
 *    channels), every channel reads and feeds the same state h_t, and the
 *    work per step grows from O(N) to O(NP).  The page's P is called R here
 *    (its intensity entry is written Theta(R)), because P names the head
 *    width of the SSD form.
 *  - metaphor-xennon "Mamba-3 next-generation architecture", section 3.3
 *    (MIMO formulation): the input enters the state through B times an
 *    input matrix and the output is C times the state.
 *  - everything else (discretisations, rotation, post-update output) as in
 *    ssm_oracle.c.
 *
 * Readings where the pages are silent (the MIMO formulas themselves were
 * lost from the first page's text): the R inputs of a channel enter through
 * the columns of B and add up in q_t; output r reads column r of C; the skip
 * term D[d] is shared by the R outputs of a channel; the trapezoid's
 * previous-input term uses q_{t-1} = sum_r B_{t-1}[n,r] u_{t-1}[r].
 *
 * Layouts, row-major in the index order of the names:
 *   u, y             : [B][L][D][R]
 *   delta, lambda    : [B][L][D]            A : [D][N]   Dskip : [D] or NULL
 *   Bm, Cm           : [B][L][N][R] (real)  or [B][L][N][R][2] (complex re,im)
 *   theta            : [B][L][D][N] or NULL
 *   h0, q0, h_last, q_last : [B][D][N] (real) or [B][D][N][2], each optional
 *   (q is the trapezoid's input term q_t defined above).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <unistd.h>

enum { MIMO_ZOH = 0, MIMO_EULER = 1, MIMO_TRAP = 2 };

typedef struct {
    double re, im;
} mc;

static mc m_make(double re, double im) {
    mc r;
    r.re = re;
    r.im = im;
    return r;
}
static mc m_add(mc a, mc b) { return m_make(a.re + b.re, a.im + b.im); }
static mc m_mul(mc a, mc b) { return m_make(a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re); }
static mc m_scale(double s, mc a) { return m_make(s * a.re, s * a.im); }

typedef struct {
    int64_t B, L, D, N, R;
    int disc, is_complex;
    const double *u, *delta, *A, *Bm, *Cm, *Dskip, *theta, *lambda, *h0, *q0;
    double *y, *h_last, *q_last;
} mimo_problem;

/* One (b, d) channel, step by step.  h, qprev: N entries; acc: R entries. */
static void mimo_channel(const mimo_problem *p, int64_t b, int64_t d, mc *h, mc *qprev, mc *acc) {
    const int64_t L = p->L, D = p->D, N = p->N, R = p->R;
    const int cw = p->is_complex ? 2 : 1;

    for (int64_t n = 0; n < N; ++n) {
        const int64_t s = ((b * D + d) * N + n) * cw;
        h[n] = p->h0 ? m_make(p->h0[s], p->is_complex ? p->h0[s + 1] : 0.0) : m_make(0.0, 0.0);
        qprev[n] = p->q0 ? m_make(p->q0[s], p->is_complex ? p->q0[s + 1] : 0.0) : m_make(0.0, 0.0);
    }
    for (int64_t t = 0; t < L; ++t) {
        const int64_t tc = (b * L + t) * D + d;
        const double dt = p->delta[tc];
        const double lam = p->disc == MIMO_TRAP ? p->lambda[tc] : 0.0;
        const double *x = p->u + tc * R; /* the channel's R inputs */
        for (int64_t r = 0; r < R; ++r) acc[r] = m_make(0.0, 0.0);

        for (int64_t n = 0; n < N; ++n) {
            const double a = p->A[d * N + n], z = dt * a, rho = exp(z);
            mc alpha = m_make(rho, 0.0);
            if (p->is_complex) {
                const double th = p->theta ? p->theta[tc * N + n] : 0.0;
                alpha = m_make(rho * cos(th), rho * sin(th));
            }
            /* q_t[n] = sum_r B[n, r] u[r] */
            const int64_t bn = ((b * L + t) * N + n) * R; /* (b, t, n, r = 0) */
            mc q = m_make(0.0, 0.0);
            for (int64_t r = 0; r < R; ++r) {
                const int64_t i = (bn + r) * cw;
                q = m_add(q, m_scale(x[r], m_make(p->Bm[i], p->is_complex ? p->Bm[i + 1] : 0.0)));
            }
            mc bterm;
            if (p->disc == MIMO_ZOH) {
                bterm = m_scale(a != 0.0 ? expm1(z) / a : dt, q);
            } else if (p->disc == MIMO_EULER) {
                bterm = m_scale(dt, q);
            } else {
                bterm = m_add(m_scale(lam * dt, q), m_scale((1.0 - lam) * dt, m_mul(alpha, qprev[n])));
            }
            qprev[n] = q;
            h[n] = m_add(m_mul(alpha, h[n]), bterm);
            /* output r reads column r of C */
            for (int64_t r = 0; r < R; ++r) {
                const int64_t i = (bn + r) * cw;
                acc[r] = m_add(acc[r], m_mul(m_make(p->Cm[i], p->is_complex ? p->Cm[i + 1] : 0.0), h[n]));
            }
        }
        const double skip = p->Dskip ? p->Dskip[d] : 0.0;
        for (int64_t r = 0; r < R; ++r) p->y[tc * R + r] = acc[r].re + skip * x[r];
    }
    for (int64_t n = 0; n < N; ++n) {
        const int64_t s = ((b * D + d) * N + n) * cw;
        if (p->h_last) {
            p->h_last[s] = h[n].re;
            if (p->is_complex) p->h_last[s + 1] = h[n].im;
        }
        if (p->q_last) {
            p->q_last[s] = qprev[n].re;
            if (p->is_complex) p->q_last[s + 1] = qprev[n].im;
        }
    }
}

typedef struct {
    const mimo_problem *p;
    int64_t begin, end; /* flattened (b, d) channels */
    int failed;
} mimo_work;

static void *mimo_worker(void *arg) {
    mimo_work *w = (mimo_work *)arg;
    mc *h = (mc *)malloc(sizeof(mc) * (size_t)w->p->N);
    mc *qp = (mc *)malloc(sizeof(mc) * (size_t)w->p->N);
    mc *acc = (mc *)malloc(sizeof(mc) * (size_t)w->p->R);
    if (!h || !qp || !acc) {
        w->failed = 1;
    } else {
        for (int64_t c = w->begin; c < w->end; ++c) mimo_channel(w->p, c / w->p->D, c % w->p->D, h, qp, acc);
    }
    free(h);
    free(qp);
    free(acc);
    return NULL;
}

/* Returns 0 on success, 1 on invalid arguments, 2 on an unsupported mode
 * (complex ZOH), 3 when threads or memory could not be obtained. */
int oracle_scan_mimo_f64(int64_t B, int64_t L, int64_t D, int64_t N, int64_t R, int disc, int is_complex,
                         const double *u, const double *delta, const double *A, const double *Bm,
                         const double *Cm, const double *Dskip, const double *theta, const double *lambda,
                         const double *h0, const double *q0, double *y, double *h_last, double *q_last,
                         int nthreads) {
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0 || R <= 0) return 1;
    if (!u || !delta || !A || !Bm || !Cm || !y) return 1;
    if (disc < MIMO_ZOH || disc > MIMO_TRAP) return 1;
    if (disc == MIMO_TRAP && !lambda) return 1;
    if (!is_complex && theta) return 1;
    if (is_complex && disc == MIMO_ZOH) return 2;

    mimo_problem p = {B, L, D, N, R, disc, is_complex, u, delta, A, Bm, Cm, Dskip, theta, lambda,
                      h0, q0, y, h_last, q_last};
    const int64_t channels = B * D;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > channels) nthreads = (int)channels;

    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    mimo_work *w = (mimo_work *)calloc((size_t)nthreads, sizeof(mimo_work));
    if (!tid || !w) {
        free(tid);
        free(w);
        return 3;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        w[i].p = &p;
        w[i].begin = channels * i / nthreads;
        w[i].end = channels * (i + 1) / nthreads;
        if (pthread_create(&tid[i], NULL, mimo_worker, &w[i]) != 0) {
            rc = 3;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(tid[i], NULL);
        if (w[i].failed) rc = 3;
    }
    free(tid);
    free(w);
    return rc;
}
