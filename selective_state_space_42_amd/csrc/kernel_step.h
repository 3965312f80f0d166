// kernel_step.h -- one step of the recurrence with the state kept in memory:
// the decode step of autoregressive generation (L = 1 per call).
//
// For every (b, d, n):  h[n] <- alpha[n] h[n] + bterm[n],  y = Re(sum_n C[n] h[n]) + D u,
// and for the trapezoid q[n] <- B[n] u (the input term the next step's beta
// multiplies).  This is the same recurrence and discretisations as the scan
// (the fengwang.github.io essay's scan section; the discretisation table of
// the ai.tomabc.com Mamba-3 story), one step at a time: recurrent inference
// carries a fixed-size state from token to token (the ai.tomabc.com story's
// motivation section and its table of inference arithmetic intensity, which
// puts this sequential step at a few operations per byte, memory-bound), and
// a state left by one call is the prefix of the next (the production
// checklist of the blog.lonae.com essay, on reusing the state).
//
// The step reads and writes the whole state, so it is bound by HBM traffic:
// per (b, d) it moves the state (and q) in and out plus the inputs.  Lanes are
// (channel, state pair): lpc lanes per channel (a power of two, 2 lpc >= N),
// two states per lane, so a channel's state is one contiguous run of memory
// read by consecutive lanes.  The sum over states is reduced by shuffles
// within the channel's lanes.
//
// Arithmetic follows the scan kernel's policies: exp(delta A) by the hardware
// 2^x; sin/cos by the hardware on fract(theta / 2 pi) for bf16 I/O and by the
// fp64-reduced polynomials for fp32 I/O; ZOH's (e^z - 1)/A by exp_expm1.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "device_math.h"

namespace ssm {

struct StepParams {
    const void* u;       // [B][D]
    const void* delta;   // [B][D]
    const float* A;      // [D][N]
    const void* B;       // [B][N] or [B][N][2]
    const void* C;       // same layout as B
    const float* Dskip;  // [D] or NULL
    const void* theta;   // [B][D][N] or NULL
    const void* lambda;  // [B][D] (trapezoid)
    float* h;            // [B][D][N] or [B][D][N][2], read and overwritten
    float* q;            // trapezoid: like h, read (q_{t-1}) and overwritten (q_t)
    void* y;             // [B][D]
    int64_t batch, dim, dstate;
    int32_t lpc;  // lanes per channel: power of two, 2 * lpc >= dstate, lpc <= 32
};

template <typename T, int DISC, bool CPLX>
__global__ void __launch_bounds__(256) scan_step_kernel(StepParams p) {
    using E = Elem<T>;
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const T* u = static_cast<const T*>(p.u);
    const T* delta = static_cast<const T*>(p.delta);
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    const T* theta = static_cast<const T*>(p.theta);
    const T* lambda = static_cast<const T*>(p.lambda);
    T* y = static_cast<T*>(p.y);

    const int lane = threadIdx.x & 63;
    const int lpc = p.lpc;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t ch = wave * (64 / lpc) + lane / lpc;  // flattened (b, d)
    const int pr = lane & (lpc - 1);                    // state pair
    const int64_t D = p.dim, N = p.dstate;
    const bool ch_ok = ch < p.batch * D;
    const int64_t b = ch_ok ? ch / D : 0;
    const int64_t d = ch_ok ? ch % D : 0;

    float x = 0.f, dt = 0.f, lam = 0.f;
    if (ch_ok) {
        x = E::load(u, ch);
        dt = E::load(delta, ch);
        if constexpr (DISC == kTrap) lam = E::load(lambda, ch);
    }
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = 2 * pr + j;
        if (!ch_ok || n >= N) continue;
        const int64_t s = ch * N + n;        // (b, d, n)
        const int64_t bn = b * N + n;        // (b, n)
        const float a = p.A[d * N + n];
        const float z = dt * a;
        float rho, em1 = 0.f;
        if constexpr (DISC == kZOH)
            exp_expm1(z, dt * prep_A(a), &rho, &em1);
        else
            rho = exp_dA(dt, prep_A(a));
        float ar = rho, ai = 0.f;
        if constexpr (CPLX) {
            if (theta) {
                float sn, cs;
                sin_cos<SC>(E::load(theta, s), &sn, &cs);
                ar = rho * cs;
                ai = rho * sn;
            }
        }
        float Br, Bi = 0.f, Cr, Ci = 0.f, hr, hi = 0.f;
        if constexpr (CPLX) {
            Br = E::load(Bm, 2 * bn);
            Bi = E::load(Bm, 2 * bn + 1);
            Cr = E::load(Cm, 2 * bn);
            Ci = E::load(Cm, 2 * bn + 1);
            hr = p.h[2 * s];
            hi = p.h[2 * s + 1];
        } else {
            Br = E::load(Bm, bn);
            Cr = E::load(Cm, bn);
            hr = p.h[s];
        }
        const float qr = Br * x, qi = Bi * x;  // q_t = B_t u_t
        float br, bi;
        if constexpr (DISC == kZOH) {
            const float coef = a != 0.f ? em1 / a : dt;
            br = coef * qr;
            bi = coef * qi;
        } else if constexpr (DISC == kEuler) {
            br = dt * qr;
            bi = dt * qi;
        } else {
            // lambda delta q_t + (1 - lambda) delta alpha_t q_{t-1}
            float pr0 = CPLX ? p.q[2 * s] : p.q[s];
            float pi0 = CPLX ? p.q[2 * s + 1] : 0.f;
            const float g = lam * dt, e = (1.f - lam) * dt;
            br = g * qr + e * (ar * pr0 - ai * pi0);
            bi = g * qi + e * (ar * pi0 + ai * pr0);
            if constexpr (CPLX) {
                p.q[2 * s] = qr;
                p.q[2 * s + 1] = qi;
            } else {
                p.q[s] = qr;
            }
        }
        const float nr = ar * hr - ai * hi + br;
        const float ni = ar * hi + ai * hr + bi;
        if constexpr (CPLX) {
            p.h[2 * s] = nr;
            p.h[2 * s + 1] = ni;
        } else {
            p.h[s] = nr;
        }
        part += Cr * nr - Ci * ni;  // Re(C h), no conjugate
    }
    for (int off = lpc >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (pr == 0 && ch_ok) E::store(y, ch, part + (p.Dskip ? p.Dskip[d] : 0.f) * x);
}

}  // namespace ssm
