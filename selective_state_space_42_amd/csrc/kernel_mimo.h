// kernel_mimo.h -- the multi-input multi-output (MIMO) scan: every (b, d)
// channel keeps one state h[n] that R inputs feed and R outputs read.
//
//   q_t[n]    = sum_r B_t[n, r] u_t[r]
//   h_t[n]    = alpha_t[n] h_{t-1}[n] + bterm_t[n]     (bterm from q_t, and
//               from q_{t-1} for the trapezoid, as in the single-input scan)
//   y_t[r]    = Re(sum_n C_t[n, r] h_t[n]) + D u_t[r]
//
// B and C are N x R per step instead of N-vectors, so the work per state and
// step grows R-fold while the state traffic stays the same (the ai.tomabc.com
// Mamba-3 story, MIMO section and its shape table; the metaphor-xennon
// Mamba-3 notes, section 3.3).  The discretisations and the rotation are
// those of the single-input scan (the same story's discretisation table and
// complex-state section).
//
// Layout of the work: one lane per (channel, state); lpc lanes per channel
// (a power of two >= max(N, R)), 64 / lpc channels per wave.  A lane reads
// its state's row of B (and C), B[b, t, n, 0..R-1], as one contiguous run,
// and the channel's R inputs as another.  The R partial sums Re(C[n, r] h[n])
// are reduced over the channel's lanes by a reduce-scatter: log2(R) halving
// levels leave one output per lane group, then the remaining levels add.
//
// Long sequences are cut into time chunks so that short, wide and long,
// narrow problems both fill the GPU:
//   mimo_scan_kernel<LOCAL>: chunks 0 .. C-2 from a zero state, keeping the
//     chunk's product of decays P = prod alpha and its end state h_loc;
//   mimo_carry_kernel: per (b, d, n), H_in(c + 1) = P_c H_in(c) + h_loc(c)
//     from H_in(0) = h0 (the combine of the fengwang.github.io essay's
//     parallel-scan section);
//   mimo_scan_kernel<OUT>: every chunk from its true incoming state, writing y
//     (and h_last, q_last from the last chunk).
// The trapezoid's q_{t0-1} at a chunk start is formed from the inputs at
// t0 - 1, so chunks need nothing from each other but the carried state.
// With one chunk the first and second kernels are skipped.
//
// Arithmetic follows the other scan kernels: exp(delta A) by the hardware
// 2^x, sin/cos by the hardware on fract(theta / 2 pi) for bf16 I/O and by the
// fp64-reduced polynomials for fp32 I/O, ZOH's (e^z - 1)/A by exp_expm1.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "device_math.h"
#include "mimo_launch.h"

namespace ssm {
namespace mimo {
constexpr int kGroup = 8;  // steps whose loads are issued together
}  // namespace mimo

// NB contiguous bytes (a power of two >= 2, naturally aligned) read with the
// widest loads that fit, kept as raw words until they are used.
template <int NB>
struct Run {
    static constexpr int kWords = NB < 4 ? 1 : NB / 4;
    uint32_t w[kWords];
};

template <int NB>
__device__ __forceinline__ void load_run(const void* p, Run<NB>& r) {
    if constexpr (NB == 2) {
        r.w[0] = *static_cast<const uint16_t*>(p);
    } else if constexpr (NB == 4) {
        r.w[0] = *static_cast<const uint32_t*>(p);
    } else if constexpr (NB == 8) {
        const uint2 v = *static_cast<const uint2*>(p);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
        static_assert(NB % 16 == 0, "runs of 2, 4, 8 or a multiple of 16 bytes");
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const uint4 v = static_cast<const uint4*>(p)[i];
            r.w[4 * i] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    }
}

// element i of a run of T values, widened exactly
template <typename T, int NB>
__device__ __forceinline__ float run_elem(const Run<NB>& r, int i) {
    if constexpr (std::is_same_v<T, float>)
        return __uint_as_float(r.w[i]);
    else
        return (i & 1) ? bf16_hi(r.w[i >> 1]) : bf16_lo(r.w[i >> 1]);
}

// The operands of one step of one lane, as loaded.
template <typename T, bool CPLX, int R>
struct MimoIn {
    static constexpr int kES = sizeof(T), kCw = CPLX ? 2 : 1;
    Run<kES> dt, lam, th;
    Run<R * kES> x;         // u[b, t, d, 0 .. R-1]
    Run<R * kCw * kES> bm;  // B[b, t, n, 0 .. R-1]
    Run<R * kCw * kES> cm;  // C[b, t, n, 0 .. R-1]
};

// q = sum_r B[r] x[r] (complex B, real x)
template <typename T, bool CPLX, int R>
__device__ __forceinline__ void mimo_q(const Run<R * (CPLX ? 2 : 1) * sizeof(T)>& bm, const float (&x)[R], float* qr,
                                       float* qi) {
    constexpr int kCw = CPLX ? 2 : 1;
    float sr = 0.f, si = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        sr = __builtin_fmaf(run_elem<T>(bm, r * kCw), x[r], sr);
        if constexpr (CPLX) si = __builtin_fmaf(run_elem<T>(bm, r * kCw + 1), x[r], si);
    }
    *qr = sr;
    *qi = si;
}

// One step of one state: alpha_t, the b-term from q_t (and q_{t-1}), and
// h <- alpha h + bterm.  Returns alpha in (ar, ai); q_{t-1} becomes q_t.
template <int DISC, bool CPLX, int SC>
__device__ __forceinline__ void mimo_advance(float dt, float lam, float th, float qr, float qi, float a, float a2,
                                             float& hr, float& hi, float& qpr, float& qpi, float* ar, float* ai) {
    float rho, em1 = 0.f;
    if constexpr (DISC == kZOH)
        exp_expm1(dt * a, dt * a2, &rho, &em1);
    else
        rho = exp_dA(dt, a2);
    float xr = rho, xi = 0.f;
    if constexpr (CPLX) {
        float sn, cs;
        sin_cos<SC>(th, &sn, &cs);
        xr = rho * cs;
        xi = rho * sn;
    }
    float br, bi;
    if constexpr (DISC == kZOH) {
        const float coef = a != 0.f ? em1 / a : dt;
        br = coef * qr;
        bi = coef * qi;
    } else if constexpr (DISC == kEuler) {
        br = dt * qr;
        bi = dt * qi;
    } else {  // lambda delta q_t + (1 - lambda) delta alpha_t q_{t-1}
        const float g = lam * dt, e = (1.f - lam) * dt;
        br = g * qr + e * (xr * qpr - xi * qpi);
        bi = g * qi + e * (xr * qpi + xi * qpr);
        qpr = qr;
        qpi = qi;
    }
    const float nr = xr * hr - xi * hi + br;
    const float ni = xr * hi + xi * hr + bi;
    hr = nr;
    hi = ni;
    *ar = xr;
    *ai = xi;
}

// Sum over the channel's lpc lanes of R partial outputs, scattered: after
// log2(R) halving levels at offsets lpc/2 .. lpc/R each lane holds the sum
// for output mimo_out_index(); the remaining levels complete it.
template <int R>
__device__ __forceinline__ float mimo_reduce_scatter(const float (&v)[R], int pr, int lpc) {
    float cur[R];
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = v[r];
    int o = lpc >> 1;
#pragma unroll
    for (int h = R / 2; h >= 1; h >>= 1) {
        const bool up = (pr & o) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float keep = up ? cur[h + i] : cur[i];
            const float send = up ? cur[i] : cur[h + i];
            cur[i] = keep + __shfl_xor(send, o, 64);
        }
        o >>= 1;
    }
    float s = cur[0];
    for (; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    return s;
}

template <int R>
__device__ __forceinline__ int mimo_out_index(int pr, int lpc) {
    int r = 0, o = lpc >> 1;
#pragma unroll
    for (int h = R / 2; h >= 1; h >>= 1) {
        if (pr & o) r += h;
        o >>= 1;
    }
    return r;
}

// x[r_own] without dynamic register indexing
template <int R>
__device__ __forceinline__ float mimo_pick(const float (&x)[R], int r_own) {
    float v = x[0];
#pragma unroll
    for (int r = 1; r < R; ++r) v = r == r_own ? x[r] : v;
    return v;
}

// Every operand of step t for one lane.  Without theta (complex state, theta
// = 0) the rotation slot reads delta's element instead and is ignored, so the
// loads carry no branches.
template <typename T, int DISC, bool CPLX, int R, bool WITH_C>
__device__ __forceinline__ void mimo_load(const MimoParams& p, int64_t b, int64_t d, int64_t n, int64_t t,
                                          MimoIn<T, CPLX, R>& in) {
    constexpr int kCw = CPLX ? 2 : 1;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t tc = (b * L + t) * D + d;
    const int64_t bn = ((b * L + t) * N + n) * R * kCw;
    const T* delta = static_cast<const T*>(p.delta);
    load_run(delta + tc, in.dt);
    if constexpr (DISC == kTrap) load_run(static_cast<const T*>(p.lambda) + tc, in.lam);
    load_run(static_cast<const T*>(p.u) + tc * R, in.x);
    if constexpr (CPLX) load_run(p.theta ? static_cast<const T*>(p.theta) + tc * N + n : delta + tc, in.th);
    load_run(static_cast<const T*>(p.B) + bn, in.bm);
    if constexpr (WITH_C) load_run(static_cast<const T*>(p.C) + bn, in.cm);
}

template <typename T, int DISC, bool CPLX, int R, bool OUT>
__global__ void __launch_bounds__(256) mimo_scan_kernel(MimoParams p) {
    constexpr int kCw = CPLX ? 2 : 1, kG = mimo::kGroup;
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const int lane = threadIdx.x & 63, lpc = p.lpc;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate, BD = p.batch * p.dim;
    const int64_t gw = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t wpc = (BD * lpc + 63) / 64;  // waves per chunk
    const int64_t c = gw / wpc;
    if (c >= (OUT ? p.nchunks : p.nchunks - 1)) return;  // whole waves
    const int64_t ch_raw = (gw % wpc) * (64 / lpc) + lane / lpc;
    const int pr = lane & (lpc - 1);
    const bool ch_ok = ch_raw < BD, ok = ch_ok && pr < N;
    // lanes past the problem compute on valid addresses and write nothing
    const int64_t ch = ch_ok ? ch_raw : BD - 1, n = pr < N ? pr : N - 1;
    const int64_t b = ch / D, d = ch % D, sidx = ch * N + n;
    const int64_t t0 = c * p.chunk, t1 = t0 + p.chunk < L ? t0 + p.chunk : L;

    const float a = p.A[d * N + n], a2 = prep_A(a);
    const float dsk = p.Dskip ? p.Dskip[d] : 0.f;
    const int r_own = mimo_out_index<R>(pr, lpc);
    const bool writer = ch_ok && (pr & (lpc / R - 1)) == 0;

    float hr = 0.f, hi = 0.f, qpr = 0.f, qpi = 0.f;
    float Pr = 1.f, Pi = 0.f;  // LOCAL: product of the chunk's decays
    if constexpr (OUT) {
        if (c == 0) {
            if (p.h0) {
                hr = p.h0[sidx * kCw];
                if constexpr (CPLX) hi = p.h0[sidx * 2 + 1];
            }
        } else {
            const float* s = p.carry + ((c - 1) * BD * N + sidx) * 2 * kCw;
            hr = s[kCw];
            if constexpr (CPLX) hi = s[3];
        }
    }
    if constexpr (DISC == kTrap) {
        if (t0 == 0) {
            if (p.q0) {
                qpr = p.q0[sidx * kCw];
                if constexpr (CPLX) qpi = p.q0[sidx * 2 + 1];
            }
        } else {  // q_{t0-1} from the inputs of step t0 - 1
            MimoIn<T, CPLX, R> in;
            mimo_load<T, DISC, CPLX, R, false>(p, b, d, n, t0 - 1, in);
            float x[R];
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = run_elem<T>(in.x, r);
            mimo_q<T, CPLX, R>(in.bm, x, &qpr, &qpi);
        }
    }
    if (!ok) hr = hi = qpr = qpi = 0.f;

    const bool has_th = CPLX && p.theta;
    T* y = static_cast<T*>(p.y);
    for (int64_t tg = t0; tg < t1; tg += kG) {
        MimoIn<T, CPLX, R> in[kG];
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            const int64_t t = tg + k < t1 ? tg + k : t1 - 1;
            mimo_load<T, DISC, CPLX, R, OUT>(p, b, d, n, t, in[k]);
        }
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            if (tg + k >= t1) break;
            const float dt = run_elem<T>(in[k].dt, 0);
            const float lam = DISC == kTrap ? run_elem<T>(in[k].lam, 0) : 0.f;
            const float th = has_th ? run_elem<T>(in[k].th, 0) : 0.f;
            float x[R];
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = run_elem<T>(in[k].x, r);
            float qr, qi;
            mimo_q<T, CPLX, R>(in[k].bm, x, &qr, &qi);
            if (!ok) qr = qi = 0.f;
            float ar, ai;
            mimo_advance<DISC, CPLX, SC>(dt, lam, th, qr, qi, a, a2, hr, hi, qpr, qpi, &ar, &ai);
            if constexpr (OUT) {
                float part[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float v = run_elem<T>(in[k].cm, r * kCw) * hr;  // Re(C h), no conjugate
                    if constexpr (CPLX) v = __builtin_fmaf(-run_elem<T>(in[k].cm, r * kCw + 1), hi, v);
                    part[r] = ok ? v : 0.f;
                }
                const float s = mimo_reduce_scatter<R>(part, pr, lpc);
                if (writer) {
                    const int64_t tc = (b * L + tg + k) * D + d;
                    Elem<T>::store(y, tc * R + r_own, s + dsk * mimo_pick<R>(x, r_own));
                }
            } else {
                const float nr = ar * Pr - ai * Pi;
                Pi = ar * Pi + ai * Pr;
                Pr = nr;
            }
        }
    }

    if (!ok) return;
    if constexpr (OUT) {
        if (c == p.nchunks - 1) {
            if (p.h_last) {
                p.h_last[sidx * kCw] = hr;
                if constexpr (CPLX) p.h_last[sidx * 2 + 1] = hi;
            }
            if (DISC == kTrap && p.q_last) {
                p.q_last[sidx * kCw] = qpr;
                if constexpr (CPLX) p.q_last[sidx * 2 + 1] = qpi;
            }
        }
    } else {
        float* s = p.carry + (c * BD * N + sidx) * 2 * kCw;
        if constexpr (CPLX)
            *reinterpret_cast<float4*>(s) = make_float4(Pr, Pi, hr, hi);
        else
            *reinterpret_cast<float2*>(s) = make_float2(Pr, hr);
    }
}

// H_in(c + 1) = P_c H_in(c) + h_loc(c) per (b, d, n), written over h_loc(c).
template <bool CPLX>
__global__ void __launch_bounds__(256) mimo_carry_kernel(MimoParams p) {
    constexpr int kCw = CPLX ? 2 : 1;
    const int64_t BDN = p.batch * p.dim * p.dstate;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= BDN) return;
    float hr = 0.f, hi = 0.f;
    if (p.h0) {
        hr = p.h0[i * kCw];
        if constexpr (CPLX) hi = p.h0[i * 2 + 1];
    }
    for (int c = 0; c + 1 < p.nchunks; ++c) {
        float* s = p.carry + (c * BDN + i) * 2 * kCw;
        if constexpr (CPLX) {
            const float4 v = *reinterpret_cast<const float4*>(s);  // (P re, P im, h re, h im)
            const float nr = v.x * hr - v.y * hi + v.z;
            hi = v.x * hi + v.y * hr + v.w;
            hr = nr;
            s[2] = hr;
            s[3] = hi;
        } else {
            const float2 v = *reinterpret_cast<const float2*>(s);
            hr = v.x * hr + v.y;
            s[1] = hr;
        }
    }
}

// One decode step of the MIMO recurrence with the state in memory.
template <typename T, int DISC, bool CPLX, int R>
__global__ void __launch_bounds__(256) mimo_step_kernel(MimoStepParams p) {
    constexpr int kCw = CPLX ? 2 : 1, kES = sizeof(T);
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const int lane = threadIdx.x & 63, lpc = p.lpc;
    const int64_t D = p.dim, N = p.dstate, BD = p.batch * p.dim;
    const int64_t gw = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t ch_raw = gw * (64 / lpc) + lane / lpc;
    const int pr = lane & (lpc - 1);
    const bool ch_ok = ch_raw < BD, ok = ch_ok && pr < N;
    const int64_t ch = ch_ok ? ch_raw : BD - 1, n = pr < N ? pr : N - 1;
    const int64_t b = ch / D, d = ch % D, sidx = ch * N + n;
    const int64_t bn = (b * N + n) * R * kCw;

    Run<kES> rdt, rlam, rth;
    Run<R * kES> rx, rxp;
    Run<R * kCw * kES> rb, rc, rbp;
    load_run(static_cast<const T*>(p.delta) + ch, rdt);
    load_run(static_cast<const T*>(p.u) + ch * R, rx);
    load_run(static_cast<const T*>(p.B) + bn, rb);
    load_run(static_cast<const T*>(p.C) + bn, rc);
    if (CPLX && p.theta) load_run(static_cast<const T*>(p.theta) + sidx, rth);
    const bool prev = DISC == kTrap && p.u_prev;
    if (DISC == kTrap) load_run(static_cast<const T*>(p.lambda) + ch, rlam);
    if (prev) {
        load_run(static_cast<const T*>(p.u_prev) + ch * R, rxp);
        load_run(static_cast<const T*>(p.B_prev) + bn, rbp);
    }
    float hr = p.h[sidx * kCw], hi = CPLX ? p.h[sidx * 2 + 1] : 0.f;
    const float a = p.A[d * N + n], a2 = prep_A(a);

    float x[R], xp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        x[r] = run_elem<T>(rx, r);
        xp[r] = prev ? run_elem<T>(rxp, r) : 0.f;
    }
    float qr, qi, qpr = 0.f, qpi = 0.f;
    mimo_q<T, CPLX, R>(rb, x, &qr, &qi);
    if (prev) mimo_q<T, CPLX, R>(rbp, xp, &qpr, &qpi);
    const float dt = run_elem<T>(rdt, 0);
    const float lam = DISC == kTrap ? run_elem<T>(rlam, 0) : 0.f;
    const float th = (CPLX && p.theta) ? run_elem<T>(rth, 0) : 0.f;
    float ar, ai;
    mimo_advance<DISC, CPLX, SC>(dt, lam, th, qr, qi, a, a2, hr, hi, qpr, qpi, &ar, &ai);
    if (ok) {
        p.h[sidx * kCw] = hr;
        if constexpr (CPLX) p.h[sidx * 2 + 1] = hi;
    }
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float v = run_elem<T>(rc, r * kCw) * hr;
        if constexpr (CPLX) v = __builtin_fmaf(-run_elem<T>(rc, r * kCw + 1), hi, v);
        part[r] = ok ? v : 0.f;
    }
    const float s = mimo_reduce_scatter<R>(part, pr, lpc);
    const int r_own = mimo_out_index<R>(pr, lpc);
    if (ch_ok && (pr & (lpc / R - 1)) == 0)
        Elem<T>::store(static_cast<T*>(p.y), ch * R + r_own,
                       s + (p.Dskip ? p.Dskip[d] : 0.f) * mimo_pick<R>(x, r_own));
}

}  // namespace ssm
