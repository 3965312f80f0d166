/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the forward selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, table or constant with
 * the HIP path.
 *
 * What it computes (the sequential definition, evaluated in IEEE binary64,
 * no fast-math, no FMA contraction):
 *
 *   for every (b, d) independently, with h_{-1}[n] = 0 and q_{-1}[n] = 0:
 *     for t = 0 .. L-1, for n = 0 .. N-1:
 *       z      = delta[b,t,d] * A[d,n]
 *       rho    = exp(z)
 *       alpha  = rho * (cos theta + i sin theta)      complex state
 *              = rho                                  real state
 *       q      = Bm[b,t,n] * u[b,t,d]
 *       bterm  = ZOH   : expm1(z)/A[d,n] * q   (limit delta*q when A = 0)
 *                EULER : delta * q
 *                TRAP  : lambda*delta*q + (1-lambda)*delta*alpha*q_{t-1}
 *       h[n]   = alpha * h[n] + bterm
 *       acc   += Cm[b,t,n] * h[n]                      (no conjugate)
 *     y[b,t,d] = Re(acc) + Dskip[d] * u[b,t,d]
 *   h_last[b,d,n] = h[n]
 *
 * Sources (page title and section; no other source is used):
 *  - recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t, the operator pair
 *    O_t = (Abar_t, Bbar_t x_t) and the combine (A2,b2)(x)(A1,b1) =
 *    (A2 A1, A2 b1 + b2): fengwang.github.io "complex parallel scan"
 *    (2026-06-14), section "the mathematical essence of the parallel scan";
 *    the same page notes that nothing in the derivation needs real numbers.
 *  - ZOH Abar = exp(dA), Bbar = (dA)^-1 (exp(dA) - I) dB: same page, section
 *    "hardware challenges" (second layer); also blog.lonae.com "dual
 *    spectral theory of SSMs 2026", section 2.1, and metaphor-xennon
 *    "Mamba-3 next-generation architecture", section 2.2.
 *  - alpha, beta, gamma of ZOH / exp-Euler / exp-trapezoidal: ai.tomabc.com
 *    Mamba-3 paper story, discretisation table (exp-trapezoidal:
 *    beta_t = (1-lambda_t) delta_t exp(delta_t A) on the previous input,
 *    gamma_t = lambda_t delta_t on the current one).
 *  - complex state with data-dependent rotation e^{i theta_t}, A real and
 *    setting only the decay: same Mamba-3 story page, complex state section.
 *  - output from the post-update state y_t = C h_t + D x_t: metaphor-xennon
 *    page section 2.2, and the mamba2_ssd loop in blog.lonae.com section 3.2.
 *
 * Readings where the pages are silent: h_{-1} = 0 and B_{-1} u_{-1} = 0 (so
 * the trapezoid's first step has no previous-input term); beta uses the
 * current step's delta_t and alpha_t (rotation included); theta is used as
 * given (e^{i theta}, not e^{i delta theta}); complex ZOH is not defined here.
 *
 * Inputs are fp64 arrays, row-major, in the index order of their names:
 *   u, delta, lambda : [B][L][D]          A      : [D][N]
 *   Bm, Cm           : [B][L][N] (real)   or [B][L][N][2] (complex re,im)
 *   Dskip            : [D] or NULL        theta  : [B][L][D][N] or NULL
 *   y                : [B][L][D]          h_last : [B][D][N] or [B][D][N][2]
 *   h0, q0 (optional): initial state / previous q, layout of h_last.
 *   q_last (optional): the last step's q = Bm u, layout of h_last.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_ZOH = 0, ORACLE_EULER = 1, ORACLE_TRAP = 2 };

typedef struct {
    double re, im;
} cplx;

static cplx c_make(double re, double im) {
    cplx r;
    r.re = re;
    r.im = im;
    return r;
}
static cplx c_add(cplx a, cplx b) { return c_make(a.re + b.re, a.im + b.im); }
static cplx c_mul(cplx a, cplx b) {
    return c_make(a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re);
}
static cplx c_scale(double s, cplx a) { return c_make(s * a.re, s * a.im); }

typedef struct {
    int64_t B, L, D, N;
    int disc, is_complex;
    const double *u, *delta, *A, *Bm, *Cm, *Dskip, *theta, *lambda;
    const double *h0, *q0;
    double *y, *h_last, *q_last;
} problem;

/* One (b, d) channel: the sequential recurrence, step by step. */
static void scan_channel(const problem *p, int64_t b, int64_t d, cplx *h, cplx *qprev) {
    const int64_t L = p->L, D = p->D, N = p->N;
    const int cw = p->is_complex ? 2 : 1; /* doubles per B/C/h entry */

    for (int64_t n = 0; n < N; ++n) {
        int64_t s = ((b * D + d) * N + n) * cw;
        h[n] = p->h0 ? c_make(p->h0[s], p->is_complex ? p->h0[s + 1] : 0.0) : c_make(0.0, 0.0);
        qprev[n] = p->q0 ? c_make(p->q0[s], p->is_complex ? p->q0[s + 1] : 0.0) : c_make(0.0, 0.0);
    }

    for (int64_t t = 0; t < L; ++t) {
        const int64_t tc = (b * L + t) * D + d;
        const double dt = p->delta[tc];
        const double x = p->u[tc];
        const double lam = (p->disc == ORACLE_TRAP) ? p->lambda[tc] : 0.0;
        cplx acc = c_make(0.0, 0.0);

        for (int64_t n = 0; n < N; ++n) {
            const double a = p->A[d * N + n];
            const double z = dt * a;
            const double rho = exp(z);
            cplx alpha;
            if (p->is_complex) {
                const double th = p->theta ? p->theta[tc * N + n] : 0.0;
                alpha = c_make(rho * cos(th), rho * sin(th));
            } else {
                alpha = c_make(rho, 0.0);
            }

            const int64_t bn = ((b * L + t) * N + n) * cw;
            const cplx Bv = c_make(p->Bm[bn], p->is_complex ? p->Bm[bn + 1] : 0.0);
            const cplx Cv = c_make(p->Cm[bn], p->is_complex ? p->Cm[bn + 1] : 0.0);
            const cplx q = c_scale(x, Bv);

            cplx bterm;
            if (p->disc == ORACLE_ZOH) {
                const double coef = (a != 0.0) ? expm1(z) / a : dt;
                bterm = c_scale(coef, q);
            } else if (p->disc == ORACLE_EULER) {
                bterm = c_scale(dt, q);
            } else {
                const cplx cur = c_scale(lam * dt, q);
                const cplx prev = c_scale((1.0 - lam) * dt, c_mul(alpha, qprev[n]));
                bterm = c_add(cur, prev);
            }
            qprev[n] = q;

            h[n] = c_add(c_mul(alpha, h[n]), bterm);
            acc = c_add(acc, c_mul(Cv, h[n]));
        }
        const double skip = p->Dskip ? p->Dskip[d] : 0.0;
        p->y[tc] = acc.re + skip * x;
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
    const problem *p;
    int64_t begin, end; /* range of flattened (b, d) channel indices */
    int failed;
} work;

static void *worker(void *arg) {
    work *w = (work *)arg;
    cplx *h = (cplx *)malloc(sizeof(cplx) * (size_t)w->p->N);
    cplx *qp = (cplx *)malloc(sizeof(cplx) * (size_t)w->p->N);
    if (!h || !qp) {
        w->failed = 1;
        free(h);
        free(qp);
        return NULL;
    }
    for (int64_t c = w->begin; c < w->end; ++c) scan_channel(w->p, c / w->p->D, c % w->p->D, h, qp);
    free(h);
    free(qp);
    return NULL;
}

/* Returns 0 on success, 1 on invalid arguments, 2 on an unsupported mode
 * (complex ZOH), 3 when threads or memory could not be obtained. */
int oracle_scan_f64(int64_t B, int64_t L, int64_t D, int64_t N, int disc, int is_complex,
                    const double *u, const double *delta, const double *A, const double *Bm,
                    const double *Cm, const double *Dskip, const double *theta,
                    const double *lambda, const double *h0, const double *q0, double *y,
                    double *h_last, double *q_last, int nthreads) {
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 1;
    if (!u || !delta || !A || !Bm || !Cm || !y) return 1;
    if (disc < ORACLE_ZOH || disc > ORACLE_TRAP) return 1;
    if (disc == ORACLE_TRAP && !lambda) return 1;
    if (!is_complex && theta) return 1;
    if (is_complex && disc == ORACLE_ZOH) return 2;

    problem p = {B, L, D, N, disc, is_complex, u, delta, A, Bm, Cm, Dskip, theta, lambda,
                 h0, q0, y, h_last, q_last};

    const int64_t channels = B * D;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > channels) nthreads = (int)channels;

    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    work *w = (work *)calloc((size_t)nthreads, sizeof(work));
    if (!tid || !w) {
        free(tid);
        free(w);
        return 3;
    }
    int rc = 0;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        w[i].p = &p;
        w[i].begin = channels * i / nthreads;
        w[i].end = channels * (i + 1) / nthreads;
        if (pthread_create(&tid[i], NULL, worker, &w[i]) != 0) {
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

/* The combine operator on n complex diagonal operators (interleaved re,im):
 *   (a2, b2) (x) (a1, b1) = (a2 a1, a2 b1 + b2)
 * where (a1, b1) is the earlier step.  fengwang.github.io "complex parallel
 * scan", section "the mathematical essence of the parallel scan". */
void oracle_combine_f64(int64_t n, const double *a2, const double *b2, const double *a1,
                        const double *b1, double *a_out, double *b_out) {
    for (int64_t i = 0; i < n; ++i) {
        const cplx A2 = c_make(a2[2 * i], a2[2 * i + 1]);
        const cplx B2 = c_make(b2[2 * i], b2[2 * i + 1]);
        const cplx A1 = c_make(a1[2 * i], a1[2 * i + 1]);
        const cplx B1 = c_make(b1[2 * i], b1[2 * i + 1]);
        const cplx ao = c_mul(A2, A1);
        const cplx bo = c_add(c_mul(A2, B1), B2);
        a_out[2 * i] = ao.re;
        a_out[2 * i + 1] = ao.im;
        b_out[2 * i] = bo.re;
        b_out[2 * i + 1] = bo.im;
    }
}
