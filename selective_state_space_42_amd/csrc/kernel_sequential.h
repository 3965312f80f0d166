// kernel_sequential.h -- the plain sequential-sweep scan kernel.
//
// One lane per (channel, state n): lanes are grouped `lpc` (a power of two
// >= N) to a channel, 64 / lpc channels per wave.  Each lane walks the whole
// sequence t = 0 .. L-1 carrying its own state h[n] in registers, so no state
// tensor is ever written to memory.  The output y_t = Re(sum_n C_t[n] h_t[n])
// + D u_t is reduced over the channel's lanes with cross-lane shuffles.
//
// The per-step update is the recurrence exactly as defined (including the
// trapezoid's previous-input term with the current alpha_t), computed in fp32
// with the device library's expf / expm1f / sincosf.  It keeps every step
// simple on purpose: this kernel is the general fallback (any N <= 64) and a
// second, independently written GPU formulation against which the chunked
// kernel can be compared.  Sources: see include/ssm_scan.h.
#pragma once

#include "device_common.h"

namespace ssm {

struct SeqParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;
    const void* theta;
    const void* lambda;
    void* y;
    float* h_last;
    const float* h0;  // state before step 0, layout of h_last (NULL: zero)
    const float* q0;  // trapezoid: q_{-1}, layout of h_last (NULL: zero)
    float* q_last;    // trapezoid: q_{L-1} (written when not NULL)
    int64_t batch, seqlen, dim, dstate;
    int32_t lpc;  // lanes per channel: power of two, dstate <= lpc <= 64
};

template <typename T, int DISC, bool CPLX>
__global__ void __launch_bounds__(256) scan_sequential_kernel(SeqParams p) {
    using E = Elem<T>;
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
    const int n = lane & (lpc - 1);
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const bool ch_ok = ch < p.batch * D;
    const bool ok = ch_ok && n < N;
    const int64_t b = ch_ok ? ch / D : 0;
    const int64_t d = ch_ok ? ch % D : 0;

    const float a = ok ? p.A[d * N + n] : 0.0f;
    const float dskip = (ch_ok && p.Dskip) ? p.Dskip[d] : 0.0f;

    const int64_t sidx = (b * D + d) * N + n;  // (b, d, n) in the layout of h_last
    float hr = 0.0f, hi = 0.0f;    // state h[n]
    float qpr = 0.0f, qpi = 0.0f;  // previous step's q = B u (trapezoid only)
    if (ok && p.h0) {
        hr = CPLX ? p.h0[2 * sidx] : p.h0[sidx];
        hi = CPLX ? p.h0[2 * sidx + 1] : 0.0f;
    }
    if (DISC == kTrap && ok && p.q0) {
        qpr = CPLX ? p.q0[2 * sidx] : p.q0[sidx];
        qpi = CPLX ? p.q0[2 * sidx + 1] : 0.0f;
    }

    for (int64_t t = 0; t < L; ++t) {
        const int64_t tc = (b * L + t) * D + d;
        float dt = 0.0f, x = 0.0f, lam = 0.0f;
        if (ch_ok) {
            dt = E::load(delta, tc);
            x = E::load(u, tc);
            if constexpr (DISC == kTrap) lam = E::load(lambda, tc);
        }
        float Br = 0.0f, Bi = 0.0f, Cr = 0.0f, Ci = 0.0f, th = 0.0f;
        if (ok) {
            const int64_t bn = (b * L + t) * N + n;
            if constexpr (CPLX) {
                Br = E::load(Bm, 2 * bn);
                Bi = E::load(Bm, 2 * bn + 1);
                Cr = E::load(Cm, 2 * bn);
                Ci = E::load(Cm, 2 * bn + 1);
                if (theta) th = E::load(theta, tc * N + n);
            } else {
                Br = E::load(Bm, bn);
                Cr = E::load(Cm, bn);
            }
        }

        const float z = dt * a;
        const float rho = expf(z);
        float ar = rho, ai = 0.0f;
        if constexpr (CPLX) {
            float s, c;
            sincosf(th, &s, &c);
            ar = rho * c;
            ai = rho * s;
        }
        const float qr = Br * x;
        const float qi = Bi * x;
        float br, bi;
        if constexpr (DISC == kZOH) {
            const float coef = (a != 0.0f) ? expm1f(z) / a : dt;
            br = coef * qr;
            bi = coef * qi;
        } else if constexpr (DISC == kEuler) {
            br = dt * qr;
            bi = dt * qi;
        } else {
            const float g = lam * dt;
            const float e = (1.0f - lam) * dt;
            const float pr = ar * qpr - ai * qpi;  // alpha_t * q_{t-1}
            const float pi = ar * qpi + ai * qpr;
            br = g * qr + e * pr;
            bi = g * qi + e * pi;
            qpr = qr;
            qpi = qi;
        }
        const float nhr = ar * hr - ai * hi + br;
        const float nhi = ar * hi + ai * hr + bi;
        hr = nhr;
        hi = nhi;

        float part = Cr * hr - Ci * hi;  // Re(C h), no conjugate
        for (int off = lpc >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (n == 0 && ch_ok) E::store(y, tc, part + dskip * x);
    }

    if (ok && p.h_last) {
        if constexpr (CPLX) {
            p.h_last[2 * sidx] = hr;
            p.h_last[2 * sidx + 1] = hi;
        } else {
            p.h_last[sidx] = hr;
        }
    }
    if (DISC == kTrap && ok && p.q_last) {  // q_{L-1}, the input term a continuation needs
        if constexpr (CPLX) {
            p.q_last[2 * sidx] = qpr;
            p.q_last[2 * sidx + 1] = qpi;
        } else {
            p.q_last[sidx] = qpr;
        }
    }
}

}  // namespace ssm
