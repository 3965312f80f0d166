// kernel_step.h -- one step of the recurrence with the state kept in memory:
// the decode step of autoregressive generation (L = 1 per call).
//
// For every (b, d, n):  h[n] <- alpha[n] h[n] + bterm[n],  y = Re(sum_n C[n] h[n]) + D u.
// The trapezoid's term for the previous step, q_{t-1}[n] = B_{t-1}[n] u_{t-1},
// is formed from the previous step's B and u (per (b, n) and per (b, d)), so
// the only per-element memory traffic is the state itself and theta.  This
// is the same recurrence and discretisations as the scan
// (the fengwang.github.io essay's scan section; the discretisation table of
// the ai.tomabc.com Mamba-3 story), one step at a time: recurrent inference
// carries a fixed-size state from token to token (the ai.tomabc.com story's
// motivation section and its table of inference arithmetic intensity, which
// puts this sequential step at a few operations per byte, memory-bound), and
// a state left by one call is the prefix of the next (the production
// checklist of the blog.lonae.com essay, on reusing the state).
//
// The step reads and writes the whole state, so it is bound by HBM traffic:
// per (b, d) it moves the state in and out plus the inputs.  Lanes are
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
    const void* u_prev;  // trapezoid: [B][D], u of the previous step (NULL: no previous step)
    const void* B_prev;  // trapezoid: like B, B of the previous step (NULL with u_prev)
    float* h;            // [B][D][N] or [B][D][N][2], read and overwritten
    void* y;             // [B][D]
    int64_t batch, dim, dstate;
    int32_t lpc;  // lanes per channel: power of two, 2 * lpc >= dstate, lpc <= 32
};

// Per-lane operands of the two states n0 = 2 pr, n0 + 1 (zeros for a state
// past N).  PAIRS: N even and every array aligned for the pair, so each array
// is read with one vector load per lane.
struct StepLane {
    float a[2], th[2], br[2], bi[2], cr[2], ci[2], pbr[2], pbi[2], hr[2], hi[2];
};

// TH: theta is given (complex state).  Every load is unconditional (a
// branch around a load makes the compiler wait for all earlier loads at the
// join): without a previous step, B_prev is read from B and masked later.
template <typename T, int DISC, bool CPLX, bool PAIRS, bool TH>
__device__ __forceinline__ void step_load(const StepParams& p, int64_t ch, int64_t b, int64_t d, int64_t n0,
                                          StepLane& v) {
    using E = Elem<T>;
    const int64_t N = p.dstate;
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    const T* Bp = static_cast<const T*>(p.B_prev ? p.B_prev : p.B);
    const T* theta = static_cast<const T*>(p.theta);
    const int64_t s = ch * N + n0, bn = b * N + n0;
    if constexpr (PAIRS) {
        const float2 a = *reinterpret_cast<const float2*>(p.A + d * N + n0);
        v.a[0] = a.x;
        v.a[1] = a.y;
        if constexpr (CPLX) {
            const float4 h = *reinterpret_cast<const float4*>(p.h + 2 * s);
            v.hr[0] = h.x, v.hi[0] = h.y, v.hr[1] = h.z, v.hi[1] = h.w;
            E::load_pair(Bm, 2 * bn, &v.br[0], &v.bi[0]);
            E::load_pair(Bm, 2 * bn + 2, &v.br[1], &v.bi[1]);
            E::load_pair(Cm, 2 * bn, &v.cr[0], &v.ci[0]);
            E::load_pair(Cm, 2 * bn + 2, &v.cr[1], &v.ci[1]);
            if constexpr (DISC == kTrap) {
                E::load_pair(Bp, 2 * bn, &v.pbr[0], &v.pbi[0]);
                E::load_pair(Bp, 2 * bn + 2, &v.pbr[1], &v.pbi[1]);
            }
            if constexpr (TH) E::load_pair(theta, s, &v.th[0], &v.th[1]);
        } else {
            const float2 h = *reinterpret_cast<const float2*>(p.h + s);
            v.hr[0] = h.x, v.hr[1] = h.y;
            E::load_pair(Bm, bn, &v.br[0], &v.br[1]);
            E::load_pair(Cm, bn, &v.cr[0], &v.cr[1]);
            if constexpr (DISC == kTrap) E::load_pair(Bp, bn, &v.pbr[0], &v.pbr[1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (n0 + j >= N) continue;
            v.a[j] = p.A[d * N + n0 + j];
            if constexpr (CPLX) {
                v.hr[j] = p.h[2 * (s + j)];
                v.hi[j] = p.h[2 * (s + j) + 1];
                v.br[j] = E::load(Bm, 2 * (bn + j));
                v.bi[j] = E::load(Bm, 2 * (bn + j) + 1);
                v.cr[j] = E::load(Cm, 2 * (bn + j));
                v.ci[j] = E::load(Cm, 2 * (bn + j) + 1);
                if constexpr (DISC == kTrap) {
                    v.pbr[j] = E::load(Bp, 2 * (bn + j));
                    v.pbi[j] = E::load(Bp, 2 * (bn + j) + 1);
                }
                if constexpr (TH) v.th[j] = E::load(theta, s + j);
            } else {
                v.hr[j] = p.h[s + j];
                v.br[j] = E::load(Bm, bn + j);
                v.cr[j] = E::load(Cm, bn + j);
                if constexpr (DISC == kTrap) v.pbr[j] = E::load(Bp, bn + j);
            }
        }
    }
}

template <typename T, int DISC, bool CPLX, bool PAIRS, bool TH>
__global__ void __launch_bounds__(256) scan_step_kernel(StepParams p) {
    using E = Elem<T>;
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const T* u = static_cast<const T*>(p.u);
    const T* delta = static_cast<const T*>(p.delta);
    const T* lambda = static_cast<const T*>(p.lambda);
    T* y = static_cast<T*>(p.y);

    const int lane = threadIdx.x & 63;
    const int lpc = p.lpc;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t ch = wave * (64 / lpc) + lane / lpc;  // flattened (b, d)
    const int pr = lane & (lpc - 1);                    // state pair
    const int64_t D = p.dim, N = p.dstate;
    const int64_t n0 = 2 * pr;
    const bool ch_ok = ch < p.batch * D;
    const bool ok = ch_ok && n0 < N;
    const int64_t b = ch_ok ? ch / D : 0;
    const int64_t d = ch_ok ? ch % D : 0;

    // per-channel inputs, unconditionally (a missing u_prev reads u, masked)
    const T* up = static_cast<const T*>(p.u_prev ? p.u_prev : p.u);
    const int64_t chc = ch_ok ? ch : 0;
    const float dsk = (p.Dskip ? p.Dskip : p.A)[d];  // masked below without D
    float x = E::load(u, chc), dt = E::load(delta, chc), lam = 0.f, xp = 0.f;
    if constexpr (DISC == kTrap) {
        lam = E::load(lambda, chc);
        xp = E::load(up, chc);
    }
    StepLane v{};
    step_load<T, DISC, CPLX, PAIRS, TH>(p, ch_ok ? ch : 0, b, d, ok ? n0 : 0, v);
    if (!ch_ok) x = dt = lam = xp = 0.f;
    if (!p.u_prev) xp = 0.f;
    const float skip = p.Dskip ? dsk : 0.f;
    if (!ok) {  // states past N (or past the channels) take no part
#pragma unroll
        for (int j = 0; j < 2; ++j)
            v.a[j] = v.th[j] = v.br[j] = v.bi[j] = v.cr[j] = v.ci[j] = v.pbr[j] = v.pbi[j] = v.hr[j] = v.hi[j] = 0.f;
    }

    float part = 0.f;
    float nr[2], ni[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float a = v.a[j];
        const float z = dt * a;
        float rho, em1 = 0.f;
        if constexpr (DISC == kZOH)
            exp_expm1(z, dt * prep_A(a), &rho, &em1);
        else
            rho = exp_dA(dt, prep_A(a));
        float ar = rho, ai = 0.f;
        if constexpr (CPLX) {
            float sn, cs;
            sin_cos<SC>(v.th[j], &sn, &cs);
            ar = rho * cs;
            ai = rho * sn;
        }
        const float qr = v.br[j] * x, qi = v.bi[j] * x;  // q_t = B_t u_t
        float br, bi;
        if constexpr (DISC == kZOH) {
            const float coef = a != 0.f ? em1 / a : dt;
            br = coef * qr;
            bi = coef * qi;
        } else if constexpr (DISC == kEuler) {
            br = dt * qr;
            bi = dt * qi;
        } else {
            // lambda delta q_t + (1 - lambda) delta alpha_t q_{t-1}, q_{t-1} = B_{t-1} u_{t-1}
            const float pr0 = v.pbr[j] * xp, pi0 = v.pbi[j] * xp;
            const float g = lam * dt, e = (1.f - lam) * dt;
            br = g * qr + e * (ar * pr0 - ai * pi0);
            bi = g * qi + e * (ar * pi0 + ai * pr0);
        }
        nr[j] = ar * v.hr[j] - ai * v.hi[j] + br;
        ni[j] = ar * v.hi[j] + ai * v.hr[j] + bi;
        part += v.cr[j] * nr[j] - v.ci[j] * ni[j];  // Re(C h), no conjugate (zero past N)
    }
    if (ok) {
        const int64_t s = ch * N + n0;
        if constexpr (PAIRS) {
            if constexpr (CPLX)
                *reinterpret_cast<float4*>(p.h + 2 * s) = make_float4(nr[0], ni[0], nr[1], ni[1]);
            else
                *reinterpret_cast<float2*>(p.h + s) = make_float2(nr[0], nr[1]);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (n0 + j >= N) continue;
                if constexpr (CPLX) {
                    p.h[2 * (s + j)] = nr[j];
                    p.h[2 * (s + j) + 1] = ni[j];
                } else {
                    p.h[s + j] = nr[j];
                }
            }
        }
    }
    for (int off = lpc >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (pr == 0 && ch_ok) E::store(y, ch, part + skip * x);
}

}  // namespace ssm
