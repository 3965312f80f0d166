// kernel_sweep.h -- the lane sweep: one lane per (channel, state), one pass
// over the whole sequence.
//
// When batch rows x channels x states give every SIMD of the GPU a few waves
// of work, the sequence needs no splitting: each lane carries its own state
// h_t[n] from t = 0 to L - 1 in registers, discretising and contracting as it
// goes.  Against the chunked kernel every element's work is done once (no
// second pass over a stored alpha_t, no aggregate sums, no look-back), and
// the kernel needs no workspace, no flags and no workgroup barriers.
//
// Work decomposition
//   lane  = (channel c, state n): 16 lanes per channel, c = lane / 16; lanes
//           with n >= N carry a zero state.
//   wave  = 4 consecutive channels of one batch row, every step.  Waves are
//           independent; a workgroup packs 4, 8 or 16 of them, each with its
//           own LDS region (a complex state's waves meet at one barrier per
//           block, so that their per-step theta pieces, adjacent in memory,
//           are read together).
//   block = 16 steps.  The wave stages the block's per-step terms in LDS,
//           sweeps the 16 steps, then sums the 16 lanes' partial outputs
//           through an LDS transpose so that lane 4 rn + rc finishes y at
//           step rn of the block for channel rc.
// Staging of a block (every load issued one block ahead, through buffer
// resources that return 0 outside the data, so ragged blocks need no branch):
//   - lane 4 rn + rc loads u, delta (the trapezoid also lambda) at step rn of
//     the block for channel rc (the trapezoid's next-step delta and lambda
//     come from the lane 4 further on; the block's last step loads them),
//     forms that (step, channel)'s terms (delta, w) once for the whole wave,
//     and keeps the output's skip term for the step it finishes;
//   - lane (c, n) loads B_t[n] and C_t[n] for steps c, c+4, c+8, c+12 (the
//     wave's four channels share them) and, for the trapezoid, the row sums
//     K_t = Re(sum_n C_t[n] B_t[n]) are formed from those with 16-lane sums;
//   - lane (c, n) loads its own theta_t[n] for the 16 steps (coalesced: a
//     wave reads 64 consecutive elements per step).
//
// The recurrence per discretisation (the discretisation table of the
// ai.tomabc.com Mamba-3 story; ZOH also section 2.1 of the blog.lonae.com
// essay), carried in fp32:
//   ZOH     h_t = e^{delta A} h_{t-1} + (e^{delta A} - 1)/A B_t u_t   (delta B_t u_t at A = 0)
//   Euler   h_t = alpha_t h_{t-1} + delta_t B_t u_t
//   trap.   carried as g_t = h_t + beta'_{t+1} B_t u_t with beta'_t = (1 - lambda_t) delta_t:
//           g_t = alpha_t g_{t-1} + (lambda_t delta_t + beta'_{t+1}) u_t B_t and
//           y_t = Re(sum_n C_t g_t) + (D - beta'_{t+1} K_t) u_t, beta'_L = 0
//           (the two-band form of the exponential-trapezoidal rule; the
//           same substitution as the chunked kernel's).
// with alpha_t = e^{delta_t A} e^{i theta_t} for a complex state (the
// complex-state section of the same story) and y_t = Re(sum_n C_t h_t) + D u_t
// from the post-update state (the mamba2_ssd loop, section 3.2 of the
// blog.lonae.com essay).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "device_math.h"

namespace ssm {

namespace sweep {
constexpr int kLPC = 16;              // lanes per channel: states n = 0 .. 15
constexpr int kCPW = 64 / kLPC;       // channels per wave
constexpr int kS = kLPC;              // steps per block (lane n finishes step n)
constexpr int kWaves = 4;             // waves per workgroup (a complex state: up to kWavesWide)
constexpr int kWavesWide = 16;        // a complex state's widest workgroup (one per CU)
constexpr int kRedStride = kS + 1;    // padded row of the output transpose
constexpr int kBcSteps = kS / kCPW;   // B/C steps loaded per lane and block
// Waves of work from which the sweep beats the chunked kernel, measured on
// MI355X (1024 SIMDs): 1.5 waves per SIMD for a real state (1536 waves: 0.22
// against 0.25 ms; 768: 0.19 against 0.15), two for a complex exp-Euler one
// (2048 waves: 0.74 against 0.89 ms), three for the complex trapezoid (its
// 2560-wave case, 2.5 per SIMD, leaves half the CUs a third workgroup and
// measured 1.60 against 1.50 ms; 3840 waves 2.02 against 2.20).
constexpr int64_t kMinWavesReal = 1536;
constexpr int64_t kMinWavesComplex = 2048;
constexpr int64_t kMinWavesComplexTrap = 3072;
constexpr int64_t kMaxStepsShort = 96;  // any shape: the sweep up to this many steps
}  // namespace sweep

struct SweepParams {
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
    const float* q0;  // trapezoid: q_{-1} = B_{-1} u_{-1}, layout of h_last (NULL: zero)
    float* q_last;    // trapezoid: q_{L-1} = B_{L-1} u_{L-1} (written when not NULL)
    int64_t batch, seqlen, dim, dstate;
};

// Waves of a launch (one per 4 channels of a batch row).
inline int64_t sweep_waves(int64_t B, int64_t D) { return B * ((D + sweep::kCPW - 1) / sweep::kCPW); }

// Whether the automatic choice takes the sweep for this shape and mode.  A
// sequence no longer than one chunked tile (96 steps) gains nothing from the
// chunked kernel's split of time and pays its extra launch; from 256 steps on
// a sweep of few waves is latency-bound (measured).
inline bool sweep_preferred(int64_t B, int64_t L, int64_t D, bool is_complex, bool trap) {
    if (L <= sweep::kMaxStepsShort) return true;
    if (!is_complex) return sweep_waves(B, D) >= sweep::kMinWavesReal;
    return sweep_waves(B, D) >= (trap ? sweep::kMinWavesComplexTrap : sweep::kMinWavesComplex);
}

// Waves per workgroup for a launch of `waves` waves on `cus` CUs.  A real
// state keeps 4 (its waves never meet).  A complex state takes the widest of
// 16, 8 and 4 that loads the busiest CU no more than 4 does: its workgroup
// reads a contiguous piece of theta per step 16 times as long as one wave's
// (8x2048x4096 complex exp-Euler fp32 1.357 -> 1.279 ms with 16, bf16 0.898
// -> 0.853 with 8), while a workgroup count that leaves CUs short of work
// costs more (4x2560x8192 trapezoid, 2560 waves: 1.54 -> 1.67 ms with 16).
inline int sweep_wg_waves(int64_t waves, bool is_complex, int cus) {
    if (!is_complex || cus < 1) return sweep::kWaves;
    auto busiest = [&](int64_t k) { return ((waves + k - 1) / k + cus - 1) / cus * k; };
    for (int k = sweep::kWavesWide; k > sweep::kWaves; k /= 2)
        if (busiest(k) <= busiest(sweep::kWaves)) return k;
    return sweep::kWaves;
}

// The per-block byte offsets a lane forms are 32-bit: 17 rows of D elements
// and 16 steps of D x N theta elements must fit.
inline bool sweep_offsets_fit(int64_t D, int64_t N, int64_t es) {
    return (sweep::kS + 1) * D * N * es * 2 < (int64_t(1) << 31);
}

// LDS of one wave.
struct SweepLds {
    float4 bc[sweep::kS][sweep::kLPC];  // (B re, B im, C re, C im) per (step, state); real: (B, C) pairs
    float2 dw[sweep::kS][sweep::kCPW];  // (delta, w) per (step, channel), two steps per 16 bytes
    float k[sweep::kS];                 // K_t (trapezoid)
    float red[64 * sweep::kRedStride];  // the lanes' partial outputs, one padded row per lane
};

// B/C entry of (step, state) in the LDS: 16 bytes for a complex state; for a
// real one the first half of the array as (B, C) pairs, the pairs of steps
// 2k and 2k+1 side by side, so that one 16-byte read serves two steps.  The
// (delta, w) terms are paired the same way: a real step then costs one LDS
// read instead of two (measured 1-3 % faster).
template <bool CPLX>
__device__ __forceinline__ void st_bc(SweepLds& s, int st, int n, const float (&v)[4]) {
    if constexpr (CPLX)
        s.bc[st][n] = make_float4(v[0], v[1], v[2], v[3]);
    else
        reinterpret_cast<float2*>(&s.bc[0][0])[((st >> 1) * sweep::kLPC + n) * 2 + (st & 1)] = make_float2(v[0], v[2]);
}
__device__ __forceinline__ float4 ld_bc_complex(const SweepLds& s, int st, int n) { return s.bc[st][n]; }

// One block's loads, as they arrive: per-(step, channel) rows for the lane's
// step, B/C entries for its kBcSteps steps.
template <typename T>
struct SweepRows {
    uint32_t x, dt, lam, dtn, lamn;  // stored bits
    float bc[sweep::kBcSteps][4];    // (B re, B im, C re, C im)
};

template <typename T>
struct SweepTheta;
template <>
struct SweepTheta<uint16_t> {
    uint32_t v[sweep::kS];
    __device__ __forceinline__ float get(int s) const { return bf16_lo(v[s]); }
    __device__ __forceinline__ float absmax() const { return 0.f; }
};
template <>
struct SweepTheta<float> {
    float v[sweep::kS];
    __device__ __forceinline__ float get(int s) const { return v[s]; }
    __device__ __forceinline__ float absmax() const {
        float m = 0.f;
#pragma unroll
        for (int s = 0; s < sweep::kS; ++s) m = fmaxf(m, fabsf(v[s]));
        return m;
    }
};

// Per-lane geometry of a wave (uniform parts in scalar registers).  A lane
// holds the state of (channel c, state n), and reads and writes the
// per-(step, channel) rows (u, delta, lambda, y) for (step rn, channel rc):
// channel-fastest, so that each quarter of the wave touches 4 channels of one
// step, one cache line, instead of one channel of 16 steps (measured 4% faster
// for a real state, 15% for the trapezoid).
struct SweepLane {
    int64_t b, d0;
    int nch, c, n, rn, rc;
    bool cok, sok, rok;
};

// Issue the per-(step, channel) and B/C loads of the block starting at step
// t0 (any t0: past the end every load returns 0).  PAIRS: B and C are aligned
// to whole complex entries, so an entry is one load.
template <typename T, int DISC, bool CPLX, bool PAIRS>
__device__ __forceinline__ void sweep_issue(const SweepParams& p, const SweepLane& g, int64_t t0, SweepRows<T>& r) {
    using namespace sweep;
    using BE = Buf<T>;
    constexpr uint32_t es = BE::kSize;
    constexpr int kCE = CPLX ? 2 : 1;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t left = L - t0 > 0 ? L - t0 : 0;
    // rows t0 .. t0 + 16 of the wave's channels (the trapezoid reads one past the block)
    {
        const int64_t rows = left > kS + 1 ? kS + 1 : left;
        const uint32_t bytes = rows ? static_cast<uint32_t>((rows - 1) * D + g.nch) * es : 0u;
        const int64_t base = rows ? (g.b * L + t0) * D + g.d0 : 0;
        const uint32_t off = g.rok ? static_cast<uint32_t>(g.rn * D + g.rc) * es : kOutOfRange;
        // the step after the block, read by the lanes of the block's last step
        // only (the others take the next step's values from a neighbour)
        const uint32_t offn = g.rok && g.rn == kS - 1 ? static_cast<uint32_t>(kS * D + g.rc) * es : kOutOfRange;
        const rsrc_t ru = make_rsrc(static_cast<const T*>(p.u) + base, bytes);
        const rsrc_t rd = make_rsrc(static_cast<const T*>(p.delta) + base, bytes);
        r.x = BE::load_raw(ru, off);
        r.dt = BE::load_raw(rd, off);
        if constexpr (DISC == kTrap) {
            const rsrc_t rl = make_rsrc(static_cast<const T*>(p.lambda) + base, bytes);
            r.lam = BE::load_raw(rl, off);
            r.dtn = BE::load_raw(rd, offn);
            r.lamn = BE::load_raw(rl, offn);
        }
    }
    // B/C entries of steps c + 4j, state n
    const int64_t steps = left > kS ? kS : left;
    const uint32_t bytes = static_cast<uint32_t>(steps * N * kCE) * es;
    const int64_t base = steps ? (g.b * L + t0) * N * kCE : 0;
    const rsrc_t rB = make_rsrc(static_cast<const T*>(p.B) + base, bytes);
    const rsrc_t rC = make_rsrc(static_cast<const T*>(p.C) + base, bytes);
    const bool nok = g.n < N;
#pragma unroll
    for (int j = 0; j < kBcSteps; ++j) {
        const int s = g.c + kCPW * j;
        const uint32_t off = nok ? static_cast<uint32_t>((s * N + g.n) * kCE) * es : kOutOfRange;
        if constexpr (!CPLX) {
            r.bc[j][0] = BE::load(rB, off);
            r.bc[j][1] = 0.f;
            r.bc[j][2] = BE::load(rC, off);
            r.bc[j][3] = 0.f;
        } else if constexpr (PAIRS) {
            BE::load_pair(rB, off, &r.bc[j][0], &r.bc[j][1]);
            BE::load_pair(rC, off, &r.bc[j][2], &r.bc[j][3]);
        } else {
            const uint32_t off1 = nok ? off + es : kOutOfRange;
            r.bc[j][0] = BE::load(rB, off);
            r.bc[j][1] = BE::load(rB, off1);
            r.bc[j][2] = BE::load(rC, off);
            r.bc[j][3] = BE::load(rC, off1);
        }
    }
}

// Where a lane's theta of the block starting at t0 lies: the resource (empty
// past the end or without theta), the lane's offset at the block's first
// step and the stride between steps.
struct SweepThetaSrc {
    rsrc_t r;
    uint32_t off, step;
};
template <typename T>
__device__ __forceinline__ SweepThetaSrc sweep_theta_src(const SweepParams& p, const SweepLane& g, int64_t t0) {
    using namespace sweep;
    constexpr uint32_t es = Buf<T>::kSize;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t left = L - t0 > 0 ? L - t0 : 0;
    const int64_t steps = left > kS ? kS : left;
    const T* theta = static_cast<const T*>(p.theta);
    const uint32_t bytes = theta && steps ? static_cast<uint32_t>(((steps - 1) * D + g.nch) * N) * es : 0u;
    const int64_t base = theta && steps ? ((g.b * L + t0) * D + g.d0) * N : 0;
    SweepThetaSrc q;
    q.r = make_rsrc(theta ? theta + base : static_cast<const T*>(p.u), bytes);
    q.off = g.sok ? static_cast<uint32_t>(g.c * N + g.n) * es : kOutOfRange;
    q.step = static_cast<uint32_t>(D * N) * es;
    return q;
}
template <typename T>
__device__ __forceinline__ void sweep_theta_load(const SweepThetaSrc& q, int st, SweepTheta<T>& th) {
    if constexpr (std::is_same_v<T, uint16_t>)
        th.v[st] = __builtin_amdgcn_raw_buffer_load_b16(q.r, q.off + st * q.step, 0, 0);
    else
        th.v[st] = Buf<float>::load(q.r, q.off + st * q.step);
}

// ZOH's decay e^z and input gain (e^z - 1)/a of one step, z = delta a
// (delta at a = 0), from delta, a, a log2(e) and 1/a (0 at a = 0).  Near
// z = 0 (|z| <= ln(2)/2) the gain is delta times the Taylor series of
// (e^z - 1)/z, with no division by a and no special case at a = 0;
// elsewhere it is (e^z - 1)/a in one fused multiply-add.  Three VALU
// instructions fewer per step than forming e^z - 1 first and dividing.
__device__ __forceinline__ void zoh_decay_gain(float dt, float a, float a_log2e, float inv_a, float* ez,
                                               float* gain) {
    constexpr float kLn2Half = 0.34657359027997264f;
    const float z = dt * a;
    float q = 1.0f / 5040.0f;
    q = q * z + 1.0f / 720.0f;
    q = q * z + 1.0f / 120.0f;
    q = q * z + 1.0f / 24.0f;
    q = q * z + 1.0f / 6.0f;
    q = q * z + 0.5f;
    q = q * z + 1.0f;  // (e^z - 1)/z to 7 terms
    const float e = __builtin_amdgcn_exp2f(dt * a_log2e);
    const bool small = fabsf(z) <= kLn2Half;
    *ez = small ? __builtin_fmaf(z, q, 1.0f) : e;
    *gain = small ? dt * q : __builtin_fmaf(e, inv_a, -inv_a);
}

// Sum of v over the 16 lanes of each row (one channel's lanes), in every
// lane of the row: DPP moves within the row (swap neighbours, swap pairs,
// mirror within each half-row, mirror the row), so no LDS round trip.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return v;
}

// Turn a block's loads into the wave's LDS terms (delta, w) per (step,
// channel); returns the skip term of y at the lane's (step rn, channel rc)
// (dsk: the skip weight of channel rc).
template <typename T, int DISC, bool CPLX>
__device__ __forceinline__ float sweep_commit(SweepLds& s, const SweepLane& g, const SweepRows<T>& r, float dsk) {
    using namespace sweep;
    using BE = Buf<T>;
    const float x = BE::widen(r.x), dt = BE::widen(r.dt);
#pragma unroll
    for (int j = 0; j < kBcSteps; ++j)
        st_bc<CPLX>(s, g.c + kCPW * j, g.n, r.bc[j]);
    float w, ey;
    if constexpr (DISC == kZOH) {
        w = x;
        ey = dsk * x;
    } else if constexpr (DISC == kEuler) {
        w = dt * x;
        ey = dsk * x;
    } else {
        // delta and lambda of the next step: those of the lane kCPW further on
        // (step rn+1 of the block, same channel), or for the block's last
        // step the row after the block, which saves two more row loads per
        // block.
        const float lam = BE::widen(r.lam);
        const float dtn_nb = __shfl_down(dt, kCPW), lamn_nb = __shfl_down(lam, kCPW);
        const bool last = g.rn == kS - 1;
        const float dtn = last ? BE::widen(r.dtn) : dtn_nb, lamn = last ? BE::widen(r.lamn) : lamn_nb;
        const float bnext = (1.f - lamn) * dtn;  // beta'_{t+1} (zero past the end)
        w = (lam * dt + bnext) * x;
        float kt[kBcSteps];
#pragma unroll
        for (int j = 0; j < kBcSteps; ++j) kt[j] = row16_sum(r.bc[j][2] * r.bc[j][0] - r.bc[j][3] * r.bc[j][1]);
        if (g.n == 0) {
#pragma unroll
            for (int j = 0; j < kBcSteps; ++j) s.k[g.c + kCPW * j] = kt[j];  // K_t = Re(sum_n C_t B_t)
        }
        ey = (dsk - bnext * s.k[g.rn]) * x;
    }
    (&s.dw[0][0])[((g.rn >> 1) * kCPW + g.rc) * 2 + (g.rn & 1)] = make_float2(dt, w);
    return ey;
}

// Sweep the 16 steps of a block from the lane's state (gr, gi), writing each
// step's partial output Re(C_t[n] g_t[n]) to the lane's row of s.red.  Once a
// step's theta is used, the same register is loaded with that step's theta
// of the next block (from `nq`).
template <typename T, int DISC, bool CPLX, int SC>
__device__ __forceinline__ void sweep_steps(SweepLds& s, const SweepLane& g, SweepTheta<T>& th,
                                            const SweepThetaSrc& nq, float a, float a2, float inv_a, float& gr,
                                            float& gi) {
    using namespace sweep;
    float* red = s.red + (g.c * kLPC + g.n) * kRedStride;
    // (delta, w) and, for a real state, (B, C) of steps 2k and 2k+1 arrive
    // in one read, one pair ahead; a complex state's B/C one step ahead
    const float4* dw4 = reinterpret_cast<const float4*>(&s.dw[0][0]);
    const float4* bc4 = reinterpret_cast<const float4*>(&s.bc[0][0]);
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 nx_dw2 = dw4[g.c], cur_dw2 = zero;
    float4 nx_bc2 = zero, cur_bc2 = zero, nx_bc = zero;
    if constexpr (CPLX)
        nx_bc = ld_bc_complex(s, 0, g.n);
    else
        nx_bc2 = bc4[g.n];
#pragma unroll
    for (int st = 0; st < kS; ++st) {
        if (st % 2 == 0) {
            cur_dw2 = nx_dw2;
            cur_bc2 = nx_bc2;
            if (st + 2 < kS) {
                nx_dw2 = dw4[((st + 2) >> 1) * kCPW + g.c];
                if constexpr (!CPLX) nx_bc2 = bc4[((st + 2) >> 1) * kLPC + g.n];
            }
        }
        const float2 dw = st % 2 ? make_float2(cur_dw2.z, cur_dw2.w) : make_float2(cur_dw2.x, cur_dw2.y);
        float4 bc;
        if constexpr (CPLX) {
            bc = nx_bc;
            if (st + 1 < kS) nx_bc = ld_bc_complex(s, st + 1, g.n);
        } else {
            bc = st % 2 ? make_float4(cur_bc2.z, 0.f, cur_bc2.w, 0.f) : make_float4(cur_bc2.x, 0.f, cur_bc2.y, 0.f);
        }

        float py;
        if constexpr (CPLX) {
            const float rho = exp_dA(dw.x, a2);
            float sn, cs;
            sin_cos<SC>(th.get(st), &sn, &cs);
            sweep_theta_load<T>(nq, st, th);
            const float ar = rho * cs, ai = rho * sn;
            const float ur = dw.y * bc.x, ui = dw.y * bc.y;
            const float nr = ar * gr - ai * gi + ur;
            const float ni = ar * gi + ai * gr + ui;
            gr = nr;
            gi = ni;
            py = bc.z * gr - bc.w * gi;
        } else {
            float rho, bt;
            if constexpr (DISC == kZOH) {
                float gain;
                zoh_decay_gain(dw.x, a, a2, inv_a, &rho, &gain);
                bt = gain * (dw.y * bc.x);
            } else {
                rho = exp_dA(dw.x, a2);
                bt = dw.y * bc.x;
            }
            gr = rho * gr + bt;
            py = bc.z * gr;
        }
        red[st] = py;
        // complex: keep the steps in order (the loads one step ahead stay
        // ahead); real: let the compiler interleave steps (measured faster)
        if constexpr (CPLX) __builtin_amdgcn_sched_barrier(0);
    }
}

// One block: commit the staged loads, issue the next block's, sweep, and
// finish the outputs of the block's 16 steps.
template <typename T, int DISC, bool CPLX, bool PAIRS>
__device__ __forceinline__ void sweep_block(const SweepParams& p, SweepLds& s, const SweepLane& g, int64_t t0,
                                            SweepRows<T>& r, SweepTheta<T>& th, float a, float a2, float inv_a,
                                            float dsr, float& gr, float& gi) {
    using namespace sweep;
    using BE = Buf<T>;
    constexpr uint32_t es = BE::kSize;
    if constexpr (CPLX) {
        // Keep the workgroup's waves in step, block by block, so that their
        // theta reads of one step (adjacent 128- or 256-byte pieces of one
        // row) reach memory together.  Nothing is exchanged: no memory wait.
        __builtin_amdgcn_s_barrier();
    }
    const float ey = sweep_commit<T, DISC, CPLX>(s, g, r, dsr);
    sweep_issue<T, DISC, CPLX, PAIRS>(p, g, t0 + kS, r);
    const SweepThetaSrc nq = sweep_theta_src<T>(p, g, t0 + kS);

    if constexpr (CPLX && std::is_same_v<T, float>) {
        // fp32 sin/cos: the polynomials when every angle of the wave's block
        // is within pi/4, else the fp64-reduced evaluation
        if (__all(th.absmax() <= kPiOver4))
            sweep_steps<T, DISC, CPLX, kSinCosPoly>(s, g, th, nq, a, a2, inv_a, gr, gi);
        else
            sweep_steps<T, DISC, CPLX, kSinCosWide>(s, g, th, nq, a, a2, inv_a, gr, gi);
    } else {
        sweep_steps<T, DISC, CPLX, kSinCosHw>(s, g, th, nq, a, a2, inv_a, gr, gi);
    }

    // sum over the channel's 16 state lanes: lane (rn, rc) takes step rn of
    // channel rc
    float acc = ey;
#pragma unroll
    for (int m = 0; m < kLPC; ++m) acc += s.red[(g.rc * kLPC + m) * kRedStride + g.rn];

    const int64_t L = p.seqlen, D = p.dim;
    const int64_t left = L - t0;
    const int64_t steps = left > kS ? kS : left;
    const uint32_t bytes = static_cast<uint32_t>((steps - 1) * D + g.nch) * es;
    const rsrc_t ry = make_rsrc(static_cast<T*>(p.y) + (g.b * L + t0) * D + g.d0, bytes);
    BE::store(ry, g.rok ? static_cast<uint32_t>(g.rn * D + g.rc) * es : kOutOfRange, acc);
}

// Workgroup i of a launch runs on XCD i mod 8.  Numbering the channel groups
// XCD by XCD (XCD x takes a contiguous run of them) puts neighbouring
// channels, which share the cache lines of the per-step rows u, delta and y,
// behind one L2.  A bijection of 0 .. nb-1 for any nb.
__device__ __forceinline__ uint32_t sweep_xcd_block(uint32_t bid, uint32_t nb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t per = (nb + kXcds - 1) / kXcds, rem = nb % kXcds;
    const uint32_t x = bid % kXcds, y = bid / kXcds;
    const uint32_t before = rem == 0 || x <= rem ? x * per : rem * per + (x - rem) * (per - 1);
    return before + y;
}

// WAVES waves per workgroup (4, 8 or 16): four waves per SIMD in each case.
template <typename T, int DISC, bool CPLX, bool PAIRS, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 16 / WAVES) sweep_scan_kernel(SweepParams p) {
    using namespace sweep;
    using E = Elem<T>;
    constexpr int kCE = CPLX ? 2 : 1;
    static_assert(WAVES == 4 || WAVES == 8 || WAVES == 16, "workgroup of 4, 8 or 16 waves");
    __shared__ SweepLds s_all[WAVES];
    // the wave index is uniform; saying so keeps every block address and
    // buffer resource in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t n_dblk = (D + kCPW - 1) / kCPW;
    // Waves past the last channel group run the same blocks with no channel
    // (every load out of range, every store dropped), so that each wave of a
    // workgroup meets the same barriers.
    const int64_t waves = p.batch * n_dblk;
    const int64_t wv = static_cast<int64_t>(sweep_xcd_block(blockIdx.x, gridDim.x)) * WAVES + wave;
    const bool live = wv < waves;
    SweepLds& s = s_all[wave];

    SweepLane g;
    g.b = live ? wv / n_dblk : 0;
    g.d0 = live ? (wv % n_dblk) * kCPW : 0;
    g.nch = live ? static_cast<int>(D - g.d0 < kCPW ? D - g.d0 : kCPW) : 0;
    g.c = lane / kLPC;
    g.n = lane % kLPC;
    g.rn = lane / kCPW;
    g.rc = lane % kCPW;
    g.cok = g.c < g.nch;
    g.sok = g.cok && g.n < N;
    g.rok = g.rc < g.nch;
    const int64_t d = g.d0 + g.c;

    const float a = g.sok ? p.A[d * N + g.n] : 0.f;
    const float a2 = prep_A(a);
    const float inv_a = a != 0.f ? 1.f / a : 0.f;
    const float dsr = g.rok && p.Dskip ? p.Dskip[g.d0 + g.rc] : 0.f;

    // initial state (the trapezoid carries g_{-1} = h_{-1} + beta'_0 q_{-1})
    const int64_t sidx = (g.b * D + d) * N + g.n;  // (b, d, n) in the layout of h_last
    float gr = 0.f, gi = 0.f;
    if (g.sok && p.h0) {
        gr = p.h0[kCE * sidx];
        if constexpr (CPLX) gi = p.h0[2 * sidx + 1];
    }
    if constexpr (DISC == kTrap) {
        if (g.sok && p.q0) {
            const int64_t tc = g.b * L * D + d;
            const float bp0 = (1.f - E::load(static_cast<const T*>(p.lambda), tc)) *
                              E::load(static_cast<const T*>(p.delta), tc);
            gr += bp0 * p.q0[kCE * sidx];
            if constexpr (CPLX) gi += bp0 * p.q0[2 * sidx + 1];
        }
    }

    SweepRows<T> r;
    SweepTheta<T> th;
    sweep_issue<T, DISC, CPLX, PAIRS>(p, g, 0, r);
    if constexpr (CPLX) {
        const SweepThetaSrc q = sweep_theta_src<T>(p, g, 0);
#pragma unroll
        for (int st = 0; st < kS; ++st) sweep_theta_load<T>(q, st, th);
    }
    for (int64_t t0 = 0; t0 < L; t0 += kS)
        sweep_block<T, DISC, CPLX, PAIRS>(p, s, g, t0, r, th, a, a2, inv_a, dsr, gr, gi);

    // the trapezoid's g_{L-1} is h_{L-1} (beta'_L = 0)
    if (g.sok && p.h_last) {
        p.h_last[kCE * sidx] = gr;
        if constexpr (CPLX) p.h_last[2 * sidx + 1] = gi;
    }
    if constexpr (DISC == kTrap) {
        if (g.sok && p.q_last) {  // q_{L-1} = B_{L-1} u_{L-1}
            const float x = E::load(static_cast<const T*>(p.u), (g.b * L + L - 1) * D + d);
            const int64_t k = (g.b * L + L - 1) * N + g.n;
            p.q_last[kCE * sidx] = E::load(static_cast<const T*>(p.B), kCE * k) * x;
            if constexpr (CPLX) p.q_last[2 * sidx + 1] = E::load(static_cast<const T*>(p.B), 2 * k + 1) * x;
        }
    }
}

}  // namespace ssm
