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
// Layout of the work: one lane per (channel, state pair); lpc lanes per
// channel (a power of two >= max(N / 2, R)), 64 / lpc channels per wave and
// 256 / lpc channels of one batch row per workgroup.  B and C, shared by a
// batch row's channels, are staged in LDS as fp32 by the whole workgroup a
// group of steps at a time, so each row is read from memory once per
// workgroup and widened once; a lane then reads each of its states' rows,
// B[b, t, n, 0..R-1], as one contiguous LDS run.  The channel's R inputs and
// the other per-channel operands are reached through pointers advanced by a
// stride per step.  The R partial sums Re(C[n, r] h[n]) are reduced over the
// channel's lanes by a reduce-scatter: log2(R) halving levels leave one
// output per lane group, then the remaining levels add.
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
constexpr int kGroup = 4;  // steps whose loads are issued together
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

// q = sum_r B[r] x[r] (complex B, real x); BT is the element type of B's run
template <typename BT, bool CPLX, int R>
__device__ __forceinline__ void mimo_q(const Run<R * (CPLX ? 2 : 1) * sizeof(BT)>& bm, const float (&x)[R], float* qr,
                                       float* qi) {
    constexpr int kCw = CPLX ? 2 : 1;
    float sr = 0.f, si = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        sr = __builtin_fmaf(run_elem<BT>(bm, r * kCw), x[r], sr);
        if constexpr (CPLX) si = __builtin_fmaf(run_elem<BT>(bm, r * kCw + 1), x[r], si);
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
// for output mimo_out_index(); the remaining levels complete it.  Which half
// a lane keeps at each level is fixed per lane: `upm` holds an all-ones word
// per halving level for the lanes that keep the upper half, and the choice
// is one bitfield select per value.
template <int R>
struct MimoUpMask {
    uint32_t m[R > 1 ? 31 - __builtin_clz(R) : 1];
};

template <int R>
__device__ __forceinline__ MimoUpMask<R> mimo_up_mask(int pr, int lpc) {
    MimoUpMask<R> u{};
    int o = lpc >> 1, l = 0;
#pragma unroll
    for (int h = R / 2; h >= 1; h >>= 1, ++l) {
        u.m[l] = (pr & o) ? ~0u : 0u;
        asm volatile("" : "+v"(u.m[l]));  // opaque: kept as a mask, not re-derived per use
        o >>= 1;
    }
    return u;
}

__device__ __forceinline__ float mimo_sel(uint32_t m, float a, float b) {  // m ? b : a, bitwise
    return __uint_as_float((__float_as_uint(b) & m) | (__float_as_uint(a) & ~m));
}

template <int R>
__device__ __forceinline__ float mimo_reduce_scatter(const float (&v)[R], const MimoUpMask<R>& up, int lpc) {
    float cur[R];
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = v[r];
    int o = lpc >> 1, l = 0;
#pragma unroll
    for (int h = R / 2; h >= 1; h >>= 1, ++l) {
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float keep = mimo_sel(up.m[l], cur[i], cur[h + i]);
            const float send = mimo_sel(up.m[l], cur[h + i], cur[i]);
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

// Per-lane pointers to one step's per-channel operands, advanced by a stride
// per step.  A lane holds two states, n0 = 2 pr and n1 = n0 + 1; a state
// past N reads state n0's element again and is masked, and a missing theta
// (complex state, theta = 0) reads delta's element instead and is ignored,
// so no load needs a branch.
template <typename T>
struct MimoPtrs {
    const T *dt, *lam, *x, *th0, *th1;
    T* y;
};

struct MimoStrides {
    int64_t tc, x, th;  // per step: delta and lambda, u and y, theta
};

template <typename T>
__device__ __forceinline__ void mimo_advance_ptrs(MimoPtrs<T>& q, const MimoStrides& s) {
    q.dt += s.tc;
    q.lam += s.tc;
    q.x += s.x;
    q.y += s.x;
    q.th0 += s.th;
    q.th1 += s.th;
}

// The per-channel operands of one step of one lane, as loaded (raw bits).
template <typename T, int R>
struct MimoIn {
    Run<sizeof(T)> dt, lam, th[2];
    Run<R * sizeof(T)> x;  // u[b, t, d, 0 .. R-1]
};

template <typename T, int DISC, bool CPLX, int R>
__device__ __forceinline__ void mimo_load(const MimoPtrs<T>& q, MimoIn<T, R>& in) {
    load_run(q.dt, in.dt);
    if constexpr (DISC == kTrap) load_run(q.lam, in.lam);
    load_run(q.x, in.x);
    if constexpr (CPLX) {
        load_run(q.th0, in.th[0]);
        load_run(q.th1, in.th[1]);
    }
}

// B and C of a group of kGroup steps, staged in LDS as fp32 by the whole
// workgroup: its channels all belong to one batch row, so they share these
// rows, and each is read from memory once per workgroup instead of once per
// wave.  A row holds E = N * R * (2 | 1) values; thread t holds values
// t + 256 i (i < kEC) of every (step, array) row between the loads and the
// LDS stores.  Rows past the chunk and values past E read zero through the
// buffer resource, so no load needs a branch.
template <typename T, bool CPLX, int R, int NA>
struct MimoStage {
    static constexpr int kEC = (64 * R * (CPLX ? 2 : 1) + 255) / 256;  // per thread and row, at N = 64
    uint32_t v[mimo::kGroup][NA][kEC];
};

template <typename T, bool CPLX, int R, int NA>
__device__ __forceinline__ void mimo_stage_load(MimoStage<T, CPLX, R, NA>& sg, const T* const (&arr)[NA],
                                                int64_t row0, int rows, int E,
                                                const uint32_t (&eoff)[MimoStage<T, CPLX, R, NA>::kEC]) {
    constexpr uint32_t es = sizeof(T);
    const uint32_t rowb = static_cast<uint32_t>(E) * es;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        const rsrc_t rs = make_rsrc(arr[a] + row0 * E, static_cast<uint32_t>(rows) * rowb);
#pragma unroll
        for (int k = 0; k < mimo::kGroup; ++k)
#pragma unroll
            for (int i = 0; i < MimoStage<T, CPLX, R, NA>::kEC; ++i)
                sg.v[k][a][i] = Buf<T>::load_raw(rs, eoff[i] + k * rowb);
    }
}

template <typename T, bool CPLX, int R, int NA>
__device__ __forceinline__ void mimo_stage_store(const MimoStage<T, CPLX, R, NA>& sg, float* sb, int E, int tid) {
#pragma unroll
    for (int k = 0; k < mimo::kGroup; ++k)
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int i = 0; i < MimoStage<T, CPLX, R, NA>::kEC; ++i) {
                const int e = tid + 256 * i;
                if (e < E) sb[(k * NA + a) * E + e] = Buf<T>::widen(sg.v[k][a][i]);
            }
}

// LDS of one workgroup: two buffers of kGroup steps x (B, C) rows of fp32.
extern __shared__ __attribute__((aligned(16))) float mimo_smem[];

// One workgroup = 256 lanes = 256 / lpc channels of one batch row and one
// time chunk; the grid covers (chunk, batch row, channel block).  The chunk
// sweep (no C, no outputs) is held to five waves per SIMD (96 VGPRs, a few
// bytes spilled), which measured 3 % faster on the whole scan than the four
// its 97 registers would give; the output sweep keeps the compiler's choice.
template <typename T, int DISC, bool CPLX, int R, bool OUT>
__global__ void __launch_bounds__(256, OUT ? 1 : 5) mimo_scan_kernel(MimoParams p) {
    constexpr int kCw = CPLX ? 2 : 1, kG = mimo::kGroup, kRun = R * kCw;
    constexpr int NA = OUT ? 2 : 1;  // staged arrays: B, and C when forming outputs
    using Stage = MimoStage<T, CPLX, R, NA>;
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lpc = p.lpc;
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate, BD = p.batch * p.dim;
    const int64_t wpr = (D * lpc + 255) / 256;  // workgroups per batch row
    const int64_t blk = blockIdx.x;
    const int64_t c = blk / (p.batch * wpr), b = (blk / wpr) % p.batch;
    const int64_t d_raw = (blk % wpr) * (256 / lpc) + wave * (64 / lpc) + lane / lpc;
    const int pr = lane & (lpc - 1);
    const int64_t n0_raw = 2 * pr;
    const bool ch_ok = d_raw < D;
    const bool ok[2] = {ch_ok && n0_raw < N, ch_ok && n0_raw + 1 < N};
    // lanes past the problem compute on valid addresses and write nothing
    const int64_t d = ch_ok ? d_raw : D - 1, n0 = n0_raw < N ? n0_raw : N - 1;
    const int64_t n1 = n0 + 1 < N ? n0 + 1 : n0;
    const int64_t ch = b * D + d;
    const int64_t s0 = ch * N + n0, s1 = ch * N + n1;  // (b, d, n) in the layout of h0
    const int64_t t0 = c * p.chunk, t1 = t0 + p.chunk < L ? t0 + p.chunk : L;
    const int E = static_cast<int>(N) * kRun;

    const float a[2] = {p.A[d * N + n0], p.A[d * N + n1]};
    const float a2[2] = {prep_A(a[0]), prep_A(a[1])};
    // the skip term D u[r] joins the sum over the channel's lanes in one lane
    const float dmask = (p.Dskip && pr == 0) ? p.Dskip[d] : 0.f;
    const int r_own = mimo_out_index<R>(pr, lpc);
    const bool writer = ch_ok && (pr & (lpc / R - 1)) == 0;
    const MimoUpMask<R> upm = mimo_up_mask<R>(pr, lpc);

    float hr[2] = {0.f, 0.f}, hi[2] = {0.f, 0.f}, qpr[2] = {0.f, 0.f}, qpi[2] = {0.f, 0.f};
    float Pr[2] = {1.f, 1.f}, Pi[2] = {0.f, 0.f};  // LOCAL: product of the chunk's decays
    const int64_t sidx[2] = {s0, s1};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if constexpr (OUT) {
            if (c == 0) {
                if (p.h0) {
                    hr[j] = p.h0[sidx[j] * kCw];
                    if constexpr (CPLX) hi[j] = p.h0[sidx[j] * 2 + 1];
                }
            } else {
                const float* sl = p.carry + ((c - 1) * BD * N + sidx[j]) * 2 * kCw;
                hr[j] = sl[kCw];
                if constexpr (CPLX) hi[j] = sl[3];
            }
        }
        if constexpr (DISC == kTrap) {
            if (t0 == 0 && p.q0) {
                qpr[j] = p.q0[sidx[j] * kCw];
                if constexpr (CPLX) qpi[j] = p.q0[sidx[j] * 2 + 1];
            }
        }
    }

    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    if (DISC == kTrap && t0 > 0) {  // q_{t0-1} from the inputs of step t0 - 1
        Run<R * sizeof(T)> rx;
        load_run(static_cast<const T*>(p.u) + ((b * L + t0 - 1) * D + d) * R, rx);
        float x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = run_elem<T>(rx, r);
        const int64_t nn[2] = {n0, n1};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            Run<kRun * sizeof(T)> rb;
            load_run(Bm + ((b * L + t0 - 1) * N + nn[j]) * kRun, rb);
            mimo_q<T, CPLX, R>(rb, x, &qpr[j], &qpi[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if (!ok[j]) hr[j] = hi[j] = qpr[j] = qpi[j] = 0.f;

    // pointers to step t0's per-channel operands
    const T* delta = static_cast<const T*>(p.delta);
    const int64_t tc0 = (b * L + t0) * D + d;
    MimoPtrs<T> q;
    q.dt = delta + tc0;
    q.lam = DISC == kTrap ? static_cast<const T*>(p.lambda) + tc0 : q.dt;
    q.x = static_cast<const T*>(p.u) + tc0 * R;
    q.y = static_cast<T*>(p.y) + tc0 * R + r_own;
    const bool has_th = CPLX && p.theta;
    q.th0 = has_th ? static_cast<const T*>(p.theta) + tc0 * N + n0 : q.dt;
    q.th1 = has_th ? q.th0 + (n1 - n0) : q.dt;
    const MimoStrides st{D, D * R, has_th ? D * N : D};

    // staging of B (and C): this thread's values of a row, and the two buffers
    const T* arr[NA];
    arr[0] = Bm;
    if constexpr (OUT) arr[NA - 1] = Cm;
    uint32_t eoff[Stage::kEC];
#pragma unroll
    for (int i = 0; i < Stage::kEC; ++i)
        eoff[i] = tid + 256 * i < E ? static_cast<uint32_t>(tid + 256 * i) * sizeof(T) : kOutOfRange;
    const int bstride = kG * NA * E;  // floats per buffer
    auto rows_at = [&](int64_t tg) { return static_cast<int>(t1 - tg < kG ? t1 - tg : kG); };
    Stage sg;
    mimo_stage_load<T, CPLX, R, NA>(sg, arr, b * L + t0, rows_at(t0), E, eoff);
    mimo_stage_store<T, CPLX, R, NA>(sg, mimo_smem, E, tid);
    __syncthreads();

    T* yp = q.y;
    // kG steps: their per-channel loads first, then their arithmetic with B
    // and C from LDS.  The tail group stops its pointers on the chunk's last
    // step, so no load passes the chunk.
    auto group = [&](int64_t tg, int boff, auto tail_tag) {
        constexpr bool kTail = decltype(tail_tag)::value;
        MimoIn<T, R> in[kG];
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            mimo_load<T, DISC, CPLX, R>(q, in[k]);
            if (!kTail || tg + k + 1 < t1) mimo_advance_ptrs(q, st);
        }
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            if (kTail && tg + k >= t1) break;
            const float* rowB = mimo_smem + boff + (k * NA) * E;
            const float dt = run_elem<T>(in[k].dt, 0);
            const float lam = DISC == kTrap ? run_elem<T>(in[k].lam, 0) : 0.f;
            float x[R];
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = run_elem<T>(in[k].x, r);
            float part[R];
#pragma unroll
            for (int r = 0; r < R; ++r) part[r] = dmask * x[r];
            const int64_t nn[2] = {n0, n1};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float th = has_th ? run_elem<T>(in[k].th[j], 0) : 0.f;
                Run<kRun * 4> bm;
                load_run(rowB + nn[j] * kRun, bm);
                float qr, qi;
                mimo_q<float, CPLX, R>(bm, x, &qr, &qi);
                if (!ok[j]) qr = qi = 0.f;
                float ar, ai;
                mimo_advance<DISC, CPLX, SC>(dt, lam, th, qr, qi, a[j], a2[j], hr[j], hi[j], qpr[j], qpi[j], &ar,
                                             &ai);
                if constexpr (OUT) {
                    Run<kRun * 4> cm;
                    load_run(rowB + E + nn[j] * kRun, cm);
#pragma unroll
                    for (int r = 0; r < R; ++r) {  // Re(C h), no conjugate; a masked state's h is 0
                        part[r] = __builtin_fmaf(run_elem<float>(cm, r * kCw), hr[j], part[r]);
                        if constexpr (CPLX) part[r] = __builtin_fmaf(-run_elem<float>(cm, r * kCw + 1), hi[j], part[r]);
                    }
                } else {
                    const float nr = ar * Pr[j] - ai * Pi[j];
                    Pi[j] = ar * Pi[j] + ai * Pr[j];
                    Pr[j] = nr;
                }
            }
            if constexpr (OUT) {
                const float sum = mimo_reduce_scatter<R>(part, upm, lpc);
                if (writer) Elem<T>::store(yp, 0, sum);
                yp += st.x;
            }
        }
    };
    // every thread runs the same groups (t0, t1 are the workgroup's), so the
    // barriers match; the next group's rows load during this group
    int buf = 0;
    for (int64_t tg = t0; tg < t1; tg += kG) {
        const bool more = tg + kG < t1;
        if (more) mimo_stage_load<T, CPLX, R, NA>(sg, arr, b * L + tg + kG, rows_at(tg + kG), E, eoff);
        if (tg + kG <= t1)
            group(tg, buf * bstride, std::false_type{});
        else
            group(tg, buf * bstride, std::true_type{});
        if (more) mimo_stage_store<T, CPLX, R, NA>(sg, mimo_smem + (buf ^ 1) * bstride, E, tid);
        __syncthreads();
        buf ^= 1;
    }

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (!ok[j]) continue;
        if constexpr (OUT) {
            if (c == p.nchunks - 1) {
                if (p.h_last) {
                    p.h_last[sidx[j] * kCw] = hr[j];
                    if constexpr (CPLX) p.h_last[sidx[j] * 2 + 1] = hi[j];
                }
                if (DISC == kTrap && p.q_last) {
                    p.q_last[sidx[j] * kCw] = qpr[j];
                    if constexpr (CPLX) p.q_last[sidx[j] * 2 + 1] = qpi[j];
                }
            }
        } else {
            float* sl = p.carry + (c * BD * N + sidx[j]) * 2 * kCw;
            if constexpr (CPLX)
                *reinterpret_cast<float4*>(sl) = make_float4(Pr[j], Pi[j], hr[j], hi[j]);
            else
                *reinterpret_cast<float2*>(sl) = make_float2(Pr[j], hr[j]);
        }
    }
}

// Bytes of LDS a mimo_scan_kernel workgroup takes: two buffers of kGroup
// steps of the B (and C) rows in fp32.
inline size_t mimo_scan_lds_bytes(int64_t dstate, int R, bool cplx, bool out) {
    return static_cast<size_t>(2 * mimo::kGroup * (out ? 2 : 1) * dstate * R * (cplx ? 2 : 1) * 4);
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

// One decode step of the MIMO recurrence with the state in memory; two
// states per lane.  A workgroup holds 256 / lpc channels of one batch row,
// whose B, C (and B_prev) rows it stages in LDS as fp32 once: each lane
// then reads its states' runs from LDS instead of every lane loading them.
// PAIRS: N even and h aligned for a lane's two states, so the state moves
// with one vector load and store per lane.
template <typename T, int DISC, bool CPLX, int R, bool PAIRS>
__global__ void __launch_bounds__(256) mimo_step_kernel(MimoStepParams p) {
    constexpr int kCw = CPLX ? 2 : 1, kES = sizeof(T), kRun = R * kCw;
    constexpr int NA = DISC == kTrap ? 3 : 2;  // staged rows: B, C (and B_prev)
    constexpr int kEC = (64 * kRun + 255) / 256;  // staged values per thread and row at N = 64
    constexpr int SC = std::is_same_v<T, uint16_t> ? kSinCosHw : kSinCosWide;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lpc = p.lpc;
    const int64_t D = p.dim, N = p.dstate;
    const int64_t wpr = (D * lpc + 255) / 256;  // workgroups per batch row
    const int64_t b = blockIdx.x / wpr;
    const int64_t d_raw = (blockIdx.x % wpr) * (256 / lpc) + wave * (64 / lpc) + lane / lpc;
    const int pr = lane & (lpc - 1);
    const int64_t n0_raw = 2 * pr;
    const bool ch_ok = d_raw < D;
    const bool ok[2] = {ch_ok && n0_raw < N, ch_ok && n0_raw + 1 < N};
    const int64_t d = ch_ok ? d_raw : D - 1, n0 = n0_raw < N ? n0_raw : N - 1;
    const int64_t n1 = n0 + 1 < N ? n0 + 1 : n0;
    const int64_t ch = b * D + d;
    const int64_t sidx[2] = {ch * N + n0, ch * N + n1};
    const int E = static_cast<int>(N) * kRun;

    // Every load is issued up front and without branches: a missing theta
    // or previous step reads delta's or this step's element instead and is
    // masked afterwards (a branch around a load would make the compiler wait
    // for all earlier loads at the join).
    const float dsk = p.Dskip ? p.Dskip[d] : 0.f;  // the one branch, before the other loads
    const T* delta = static_cast<const T*>(p.delta);
    const T* uu = static_cast<const T*>(p.u);
    const bool has_th = CPLX && p.theta;
    const bool prev = DISC == kTrap && p.u_prev;
    const T* thp = has_th ? static_cast<const T*>(p.theta) : nullptr;
    const T* upp = prev ? static_cast<const T*>(p.u_prev) : uu;
    // the batch row's B, C (and B_prev; B when there is no previous step,
    // whose term is masked) through buffer resources: values past E read 0
    const T* rows[3] = {static_cast<const T*>(p.B), static_cast<const T*>(p.C),
                        prev ? static_cast<const T*>(p.B_prev) : static_cast<const T*>(p.B)};
    uint32_t sv[NA][kEC];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        const rsrc_t rs = make_rsrc(rows[a] + b * E, static_cast<uint32_t>(E) * kES);
#pragma unroll
        for (int i = 0; i < kEC; ++i) {
            const int e = tid + 256 * i;
            sv[a][i] = Buf<T>::load_raw(rs, e < E ? static_cast<uint32_t>(e) * kES : kOutOfRange);
        }
    }
    Run<kES> rdt, rlam, rth[2];
    Run<R * kES> rx, rxp;
    load_run(delta + ch, rdt);
    load_run(uu + ch * R, rx);
    if constexpr (DISC == kTrap) {
        load_run(static_cast<const T*>(p.lambda) + ch, rlam);
        load_run(upp + ch * R, rxp);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if constexpr (CPLX) load_run(has_th ? thp + sidx[j] : delta + ch, rth[j]);
    const float a_n[2] = {p.A[d * N + n0], p.A[d * N + n1]};
    float hr[2], hi[2] = {0.f, 0.f};
    if constexpr (PAIRS) {
        if constexpr (CPLX) {
            const float4 v = *reinterpret_cast<const float4*>(p.h + sidx[0] * 2);
            hr[0] = v.x, hi[0] = v.y, hr[1] = v.z, hi[1] = v.w;
        } else {
            const float2 v = *reinterpret_cast<const float2*>(p.h + sidx[0]);
            hr[0] = v.x, hr[1] = v.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            hr[j] = p.h[sidx[j] * kCw];
            if constexpr (CPLX) hi[j] = p.h[sidx[j] * 2 + 1];
        }
    }
    // stage the rows (widened) and wait for the whole workgroup's
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int i = 0; i < kEC; ++i) {
            const int e = tid + 256 * i;
            if (e < E) mimo_smem[a * E + e] = Buf<T>::widen(sv[a][i]);
        }
    __syncthreads();

    float x[R], xp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        x[r] = run_elem<T>(rx, r);
        xp[r] = prev ? run_elem<T>(rxp, r) : 0.f;
    }
    const float dt = run_elem<T>(rdt, 0);
    const float lam = DISC == kTrap ? run_elem<T>(rlam, 0) : 0.f;
    float part[R];
    const float dmask = pr == 0 ? dsk : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = dmask * x[r];
    const int64_t nn[2] = {n0, n1};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        Run<kRun * 4> rb, rc;
        load_run(mimo_smem + nn[j] * kRun, rb);
        load_run(mimo_smem + E + nn[j] * kRun, rc);
        float qr, qi, qpr = 0.f, qpi = 0.f;
        mimo_q<float, CPLX, R>(rb, x, &qr, &qi);
        if constexpr (DISC == kTrap) {  // zero without a previous step (xp = 0)
            Run<kRun * 4> rbp;
            load_run(mimo_smem + 2 * E + nn[j] * kRun, rbp);
            mimo_q<float, CPLX, R>(rbp, xp, &qpr, &qpi);
        }
        const float a = a_n[j];
        const float th = has_th ? run_elem<T>(rth[j], 0) : 0.f;
        float ar, ai;
        mimo_advance<DISC, CPLX, SC>(dt, lam, th, qr, qi, a, prep_A(a), hr[j], hi[j], qpr, qpi, &ar, &ai);
        if (!ok[j]) hr[j] = hi[j] = 0.f;  // a masked state adds nothing below
#pragma unroll
        for (int r = 0; r < R; ++r) {
            part[r] = __builtin_fmaf(run_elem<float>(rc, r * kCw), hr[j], part[r]);
            if constexpr (CPLX) part[r] = __builtin_fmaf(-run_elem<float>(rc, r * kCw + 1), hi[j], part[r]);
        }
    }
    if constexpr (PAIRS) {
        if (ok[0]) {
            if constexpr (CPLX)
                *reinterpret_cast<float4*>(p.h + sidx[0] * 2) = make_float4(hr[0], hi[0], hr[1], hi[1]);
            else
                *reinterpret_cast<float2*>(p.h + sidx[0]) = make_float2(hr[0], hr[1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!ok[j]) continue;
            p.h[sidx[j] * kCw] = hr[j];
            if constexpr (CPLX) p.h[sidx[j] * 2 + 1] = hi[j];
        }
    }
    const float sum = mimo_reduce_scatter<R>(part, mimo_up_mask<R>(pr, lpc), lpc);
    const int r_own = mimo_out_index<R>(pr, lpc);
    if (ch_ok && (pr & (lpc / R - 1)) == 0) Elem<T>::store(static_cast<T*>(p.y), ch * R + r_own, sum);
}

// Bytes of LDS a mimo_step_kernel workgroup takes: the B, C (and B_prev)
// rows of one batch row in fp32.
inline size_t mimo_step_lds_bytes(int64_t dstate, int R, bool cplx, bool trap) {
    return static_cast<size_t>((trap ? 3 : 2) * dstate * R * (cplx ? 2 : 1) * 4);
}

}  // namespace ssm
