/*
 * ssm_oracle_bwd.c -- plain fp64 CPU oracle for the gradients of the
 * selective scan (reverse mode of the sequential definition).
 *
 * TEST INFRASTRUCTURE ONLY, like ssm_oracle.c: nothing in the product
 * library links, loads or calls this file, and it shares no code with the
 * HIP path.
 *
 * The forward computation is the one in ssm_oracle.c (same page sources):
 *   z = delta_t A[d,n], alpha_t = e^z e^{i theta_t} (real: e^z),
 *   q_t = Bm_t u_t, h_t = alpha_t h_{t-1} + bterm_t, y_t = Re sum_n Cm_t h_t + D u_t,
 *   bterm: ZOH kappa q_t with kappa = expm1(z)/A (delta when A = 0);
 *          EULER delta q_t; TRAP lambda delta q_t + (1 - lambda) delta alpha_t q_{t-1}.
 * Given dy = dL/dy and dh_last = dL/dh_last, this file returns dL/d(every
 * input) for the scalar L = sum dy*y + <dh_last, h_last>.
 *
 * Convention for complex quantities: the gradient of a complex value v is
 * G = dL/dRe(v) + i dL/dIm(v), stored (re, im) like v.  With it, for
 * v = a*w (complex product) the chain rule reads dw += conj(a) G, and
 * dL = Re(conj(G) dv).  The reverse sweep, per (b, d), from t = L-1 down to 0:
 *   G_t    = dy_t conj(C_t) + conj(alpha_{t+1}) G_{t+1}      (G_L = dh_last)
 *   dC_t  += dy_t conj(h_t);  dD += dy_t u_t;  du_t += dy_t D
 *   dalpha = conj(h_{t-1}) G_t;  dbterm = G_t
 *   then each bterm form and q_t = B_t u_t by the product rule, and
 *   alpha = exp(z + i theta):  dz = Re(conj(dalpha) alpha),
 *                              dtheta = -Im(conj(dalpha) alpha),
 *   z = delta A:  ddelta += dz A,  dA += dz delta.
 * The trapezoid's term on q_{t-1} sends (1 - lambda_t) delta_t conj(alpha_t)
 * dbterm_t back to step t-1's q.  dh0 = G_{-1}, the gradient of the state
 * before step 0.
 *
 * ZOH's kappa(delta, A) = expm1(delta A)/A has d kappa/d delta = e^z and
 * d kappa/d A = (delta e^z - kappa)/A, which cancels for small z; there the
 * Taylor series delta^2 (1/2 + z/3 + z^2/8 + z^3/30) is used (|z| < 1e-4,
 * truncation below 1e-17 relative).
 *
 * Layouts are those of ssm_oracle.c; gradients have the layout of their
 * input (dB, dC complex (re, im)); dA, dB, dC, dD sum over every channel,
 * batch row and step that uses them.  Single-threaded (the sums over
 * channels need no synchronisation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    double re, im;
} bc;

static bc b_make(double re, double im) {
    bc r;
    r.re = re;
    r.im = im;
    return r;
}
static bc b_add(bc a, bc b) { return b_make(a.re + b.re, a.im + b.im); }
static bc b_mul(bc a, bc b) { return b_make(a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re); }
static bc b_conj(bc a) { return b_make(a.re, -a.im); }
static bc b_scale(double s, bc a) { return b_make(s * a.re, s * a.im); }
/* Re(conj(a) b), the real inner product of two complex numbers */
static double b_dot(bc a, bc b) { return a.re * b.re + a.im * b.im; }

enum { BW_ZOH = 0, BW_EULER = 1, BW_TRAP = 2 };

/* Returns 0 on success, 1 on invalid arguments, 2 on an unsupported mode,
 * 3 when memory could not be obtained. */
int oracle_scan_bwd_f64(int64_t B, int64_t L, int64_t D, int64_t N, int disc, int is_complex,
                        const double *u, const double *delta, const double *A, const double *Bm,
                        const double *Cm, const double *Dskip, const double *theta,
                        const double *lambda, const double *h0, const double *dy,
                        const double *dh_last, double *du, double *ddelta, double *dA, double *dB,
                        double *dC, double *dD, double *dtheta, double *dlambda, double *dh0) {
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 1;
    if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC) return 1;
    if (disc < BW_ZOH || disc > BW_TRAP) return 1;
    if (disc == BW_TRAP && (!lambda || !dlambda)) return 1;
    if (!is_complex && theta) return 1;
    if (is_complex && disc == BW_ZOH) return 2;
    const int cw = is_complex ? 2 : 1;

    /* per channel: h_t for t = -1 .. L-1, alpha_t and q_t for t = 0 .. L-1 */
    bc *hs = (bc *)malloc(sizeof(bc) * (size_t)((L + 1) * N));
    bc *al = (bc *)malloc(sizeof(bc) * (size_t)(L * N));
    bc *qs = (bc *)malloc(sizeof(bc) * (size_t)(L * N));
    bc *G = (bc *)malloc(sizeof(bc) * (size_t)N);
    bc *dqc = (bc *)malloc(sizeof(bc) * (size_t)N);
    if (!hs || !al || !qs || !G || !dqc) {
        free(hs), free(al), free(qs), free(G), free(dqc);
        return 3;
    }
    memset(dA, 0, sizeof(double) * (size_t)(D * N));
    memset(dB, 0, sizeof(double) * (size_t)(B * L * N * cw));
    memset(dC, 0, sizeof(double) * (size_t)(B * L * N * cw));
    if (dD) memset(dD, 0, sizeof(double) * (size_t)D);

    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            /* forward sweep, keeping every state */
            for (int64_t n = 0; n < N; ++n) {
                const int64_t s = ((b * D + d) * N + n) * cw;
                hs[n] = h0 ? b_make(h0[s], is_complex ? h0[s + 1] : 0.0) : b_make(0.0, 0.0);
            }
            for (int64_t t = 0; t < L; ++t) {
                const int64_t tc = (b * L + t) * D + d;
                const double dt = delta[tc], x = u[tc];
                const double lam = disc == BW_TRAP ? lambda[tc] : 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = A[d * N + n], z = dt * a, rho = exp(z);
                    const double th = theta ? theta[tc * N + n] : 0.0;
                    const bc alpha = is_complex ? b_make(rho * cos(th), rho * sin(th)) : b_make(rho, 0.0);
                    const int64_t bn = ((b * L + t) * N + n) * cw;
                    const bc q = b_scale(x, b_make(Bm[bn], is_complex ? Bm[bn + 1] : 0.0));
                    bc bt;
                    if (disc == BW_ZOH) {
                        bt = b_scale(a != 0.0 ? expm1(z) / a : dt, q);
                    } else if (disc == BW_EULER) {
                        bt = b_scale(dt, q);
                    } else {
                        const bc qp = t > 0 ? qs[(t - 1) * N + n] : b_make(0.0, 0.0);
                        bt = b_add(b_scale(lam * dt, q), b_scale((1.0 - lam) * dt, b_mul(alpha, qp)));
                    }
                    al[t * N + n] = alpha;
                    qs[t * N + n] = q;
                    hs[(t + 1) * N + n] = b_add(b_mul(alpha, hs[t * N + n]), bt);
                }
            }

            /* reverse sweep */
            for (int64_t n = 0; n < N; ++n) {
                const int64_t s = ((b * D + d) * N + n) * cw;
                G[n] = dh_last ? b_make(dh_last[s], is_complex ? dh_last[s + 1] : 0.0) : b_make(0.0, 0.0);
                dqc[n] = b_make(0.0, 0.0);
            }
            const double skip = Dskip ? Dskip[d] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t tc = (b * L + t) * D + d;
                const double dt = delta[tc], x = u[tc], g = dy[tc];
                const double lam = disc == BW_TRAP ? lambda[tc] : 0.0;
                double gu = g * skip, gdt = 0.0, glam = 0.0;
                if (dD) dD[d] += g * x;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = A[d * N + n], z = dt * a;
                    const int64_t bn = ((b * L + t) * N + n) * cw;
                    const bc Bv = b_make(Bm[bn], is_complex ? Bm[bn + 1] : 0.0);
                    const bc Cv = b_make(Cm[bn], is_complex ? Cm[bn + 1] : 0.0);
                    const bc alpha = al[t * N + n], q = qs[t * N + n];
                    const bc ht = hs[(t + 1) * N + n], hp = hs[t * N + n];

                    /* y_t = Re(C h_t) + D u_t */
                    G[n] = b_add(G[n], b_scale(g, b_conj(Cv)));
                    const bc gC = b_scale(g, b_conj(ht));
                    dC[bn] += gC.re;
                    if (is_complex) dC[bn + 1] += gC.im;

                    /* h_t = alpha h_{t-1} + bterm */
                    bc galpha = b_mul(b_conj(hp), G[n]);
                    const bc gb = G[n];
                    bc gq = dqc[n]; /* from step t+1's trapezoid term on q_t */
                    double gz = 0.0;
                    if (disc == BW_ZOH) {
                        const double kappa = a != 0.0 ? expm1(z) / a : dt;
                        gq = b_add(gq, b_scale(kappa, gb));
                        const double gk = b_dot(gb, q);
                        double dk_da;
                        if (fabs(z) < 1e-4)
                            dk_da = dt * dt * (0.5 + z * (1.0 / 3.0 + z * (1.0 / 8.0 + z * (1.0 / 30.0))));
                        else
                            dk_da = (dt * exp(z) - kappa) / a;
                        gdt += gk * exp(z);
                        dA[d * N + n] += gk * dk_da;
                    } else if (disc == BW_EULER) {
                        gq = b_add(gq, b_scale(dt, gb));
                        gdt += b_dot(gb, q);
                    } else {
                        const bc qp = t > 0 ? qs[(t - 1) * N + n] : b_make(0.0, 0.0);
                        const bc aqp = b_mul(alpha, qp);
                        gq = b_add(gq, b_scale(lam * dt, gb));
                        glam += b_dot(gb, b_add(b_scale(dt, q), b_scale(-dt, aqp)));
                        gdt += b_dot(gb, b_add(b_scale(lam, q), b_scale(1.0 - lam, aqp)));
                        galpha = b_add(galpha, b_mul(b_conj(b_scale((1.0 - lam) * dt, qp)), gb));
                        dqc[n] = b_mul(b_conj(b_scale((1.0 - lam) * dt, alpha)), gb); /* to q_{t-1} */
                    }

                    /* q_t = B_t u_t */
                    dB[bn] += x * gq.re;
                    if (is_complex) dB[bn + 1] += x * gq.im;
                    gu += b_dot(gq, Bv);

                    /* alpha = exp(z + i theta) */
                    const bc P = b_mul(b_conj(galpha), alpha);
                    gz += P.re;
                    if (dtheta) dtheta[tc * N + n] = -P.im;
                    gdt += gz * a;
                    dA[d * N + n] += gz * dt;

                    /* to h_{t-1} */
                    G[n] = b_mul(b_conj(alpha), G[n]);
                }
                du[tc] = gu;
                ddelta[tc] = gdt;
                if (disc == BW_TRAP) dlambda[tc] = glam;
            }
            if (dh0) {
                for (int64_t n = 0; n < N; ++n) {
                    const int64_t s = ((b * D + d) * N + n) * cw;
                    dh0[s] = G[n].re;
                    if (is_complex) dh0[s + 1] = G[n].im;
                }
            }
        }
    }
    free(hs), free(al), free(qs), free(G), free(dqc);
    return 0;
}
