// kernel_ssd.h -- the state-space dual (SSD) form of the scan for heads with
// a scalar decay, as matrix products on the MFMA units.
//
// The setting (blog.lonae.com essay on the dual spectral theory of SSMs,
// section 3, "Mamba-2's SSD duality"): A is a scalar per head (A = a I), so
// every state of every channel of a head decays by the same
// alpha_t = exp(delta_t a) per step, with delta_t one value per (b, t, head).
// With the exponential-Euler b-term the recurrence of channel d in head h is
//   h_t[n] = alpha_t h_{t-1}[n] + delta_t B_t[n] u_t[d],
//   y_t[d] = sum_n C_t[n] h_t[n] + D[d] u_t[d],
// the scan of include/ssm_scan.h with delta and A broadcast over the head.
// The same section shows this recurrence is a masked (causal, decaying)
// linear attention, y = (L o (C B^T)) X: over a chunk of Q steps, with
// cum_t = sum_{r <= t} delta_r a inside the chunk,
//   Y[t, p]   = sum_{s <= t} exp(cum_t - cum_s) (C_t . B_s) delta_s X[s, p]   (intra-chunk)
//             + exp(cum_t) sum_n C_t[n] H_in[n, p]                            (state entering the chunk)
//   H_out     = exp(cum_{Q-1}) H_in + sum_s exp(cum_{Q-1} - cum_s) delta_s B_s X[s, :]
// The intra-chunk product (Q x Q) . (Q x P) is a dense contraction: it runs
// on the bf16 MFMA units (v_mfma_f32_32x32x8_bf16, fp32 accumulation); the
// small terms over N run on the vector units.
//
// Three kernels (per batch row b and head h, chunks of Q = 64 steps, heads of
// P = 64 channels):
//   ssd_state_kernel  each chunk's local state contribution S_c (N x P) and
//                     its decay e_c = exp(cum_{Q-1}), all chunks in parallel;
//   ssd_pass_kernel   the states entering each chunk, H_in(c+1) = e_c H_in(c)
//                     + S_c, one thread per state element walking the chunks;
//   ssd_out_kernel    each chunk's outputs from its inputs and H_in(c).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace ssm {

namespace ssd {
constexpr int kQ = 64;      // steps per chunk
constexpr int kP = 64;      // channels per head
constexpr int kMaxN = 64;   // states
constexpr int kPad = 8;     // bf16 row padding of the MFMA operand tiles
}  // namespace ssd

struct SsdParams {
    const void* u;      // [B][L][D]
    const void* delta;  // [B][L][H]
    const float* A;     // [H]
    const void* B;      // [B][L][N]
    const void* C;      // [B][L][N]
    const float* Dskip; // [D] or NULL
    void* y;            // [B][L][D]
    float* h_last;      // [B][D][N] or NULL
    float* S;           // [B][H][nC][N][P]  chunk contributions (workspace)
    float* E;           // [B][H][nC]        chunk decays (workspace)
    float* Hin;         // [B][H][nC][N][P]  state entering each chunk (workspace)
    int64_t batch, seqlen, dim, dstate, heads, nchunks;
};

// Inclusive prefix sum of s[0 .. kQ) in place by one wave (lanes 0 .. 63).
__device__ __forceinline__ void ssd_cumsum_wave(float* s, int lane) {
    float v = s[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    s[lane] = v;
}

template <typename T>
__global__ void __launch_bounds__(256) ssd_state_kernel(SsdParams p) {
    using namespace ssd;
    using E = Elem<T>;
    const int tid = threadIdx.x;
    const int64_t nC = p.nchunks, H = p.heads, L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t c = blockIdx.x % nC, bh = blockIdx.x / nC, b = bh / H, h = bh % H;
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    __shared__ float s_x[kQ][kP + 1];
    __shared__ float s_b[kQ][kMaxN + 1];
    __shared__ float s_cum[kQ], s_w[kQ];
    const T* u = static_cast<const T*>(p.u);
    const T* Bm = static_cast<const T*>(p.B);
    const T* dl = static_cast<const T*>(p.delta);
    for (int i = tid; i < kQ * kP; i += 256) {
        const int t = i / kP, pp = i % kP;
        s_x[t][pp] = t < len ? E::load(u, (b * L + t0 + t) * D + h * kP + pp) : 0.f;
    }
    for (int i = tid; i < kQ * N; i += 256) {
        const int t = static_cast<int>(i / N), n = static_cast<int>(i % N);
        s_b[t][n] = t < len ? E::load(Bm, (b * L + t0 + t) * N + n) : 0.f;
    }
    const float a = p.A[h];
    if (tid < kQ) {
        const float dt = tid < len ? E::load(dl, (b * L + t0 + tid) * H + h) : 0.f;
        s_w[tid] = dt;
        s_cum[tid] = dt * a;
        ssd_cumsum_wave(s_cum, tid);
    }
    __syncthreads();
    const float last = s_cum[kQ - 1];
    if (tid < kQ) s_w[tid] *= expf(last - s_cum[tid]);  // exp(cum_{Q-1} - cum_s) delta_s
    __syncthreads();
    float* S = p.S + (bh * nC + c) * N * kP;
    for (int i = tid; i < N * kP; i += 256) {
        const int n = i / kP, pp = i % kP;
        float acc = 0.f;
#pragma unroll 8
        for (int t = 0; t < kQ; ++t) acc = fmaf(s_b[t][n] * s_w[t], s_x[t][pp], acc);
        S[i] = acc;
    }
    if (tid == 0) p.E[bh * nC + c] = expf(last);
}

__global__ void __launch_bounds__(256) ssd_pass_kernel(SsdParams p) {
    using namespace ssd;
    const int64_t nC = p.nchunks, H = p.heads, N = p.dstate;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // (b, h, n, pp)
    if (i >= p.batch * H * N * kP) return;
    const int64_t bh = i / (N * kP), np = i % (N * kP);
    const float* S = p.S + bh * nC * N * kP + np;
    float* Hin = p.Hin + bh * nC * N * kP + np;
    const float* E = p.E + bh * nC;
    float st = 0.f;
    int64_t c = 0;
    // eight chunks' loads at a time, then the dependent chain over them
    for (; c + 8 <= nC; c += 8) {
        float s[8], e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s[k] = S[(c + k) * N * kP];
            e[k] = E[c + k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            Hin[(c + k) * N * kP] = st;
            st = fmaf(e[k], st, s[k]);
        }
    }
    for (; c < nC; ++c) {
        Hin[c * N * kP] = st;
        st = fmaf(E[c], st, S[c * N * kP]);
    }
    if (p.h_last) {
        const int64_t b = bh / H, h = bh % H, n = np / kP, pp = np % kP;
        p.h_last[(b * p.dim + h * kP + pp) * N + n] = st;
    }
}

typedef short ssd_bf16x4 __attribute__((ext_vector_type(4)));
typedef float ssd_f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
__global__ void __launch_bounds__(256) ssd_out_kernel(SsdParams p) {
    using namespace ssd;
    using E = Elem<T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nC = p.nchunks, H = p.heads, L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t c = blockIdx.x % nC, bh = blockIdx.x / nC, b = bh / H, h = bh % H;
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    // MFMA operands in bf16: M = (C B^T) o decay o delta (rows t, columns s) and
    // X transposed (rows p, columns s), so each lane's 4 consecutive k values
    // are one 8-byte LDS read
    __shared__ __align__(16) uint16_t s_m[kQ][kQ + kPad];
    __shared__ __align__(16) uint16_t s_xt[kP][kQ + kPad];
    __shared__ float s_c[kQ][kMaxN + 1];
    __shared__ float s_b[kQ][kMaxN + 1];
    __shared__ float s_h[kMaxN][kP + 1];
    __shared__ float s_cum[kQ], s_dt[kQ];
    const T* u = static_cast<const T*>(p.u);
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    const T* dl = static_cast<const T*>(p.delta);
    for (int i = tid; i < kQ * kP; i += 256) {
        const int t = i / kP, pp = i % kP;
        const float x = t < len ? E::load(u, (b * L + t0 + t) * D + h * kP + pp) : 0.f;
        s_xt[pp][t] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // exact for bf16 input
    }
    for (int i = tid; i < kQ * N; i += 256) {
        const int t = static_cast<int>(i / N), n = static_cast<int>(i % N);
        const bool ok = t < len;
        s_b[t][n] = ok ? E::load(Bm, (b * L + t0 + t) * N + n) : 0.f;
        s_c[t][n] = ok ? E::load(Cm, (b * L + t0 + t) * N + n) : 0.f;
    }
    const float* Hin = p.Hin + (bh * nC + c) * N * kP;
    for (int i = tid; i < N * kP; i += 256) s_h[i / kP][i % kP] = Hin[i];
    const float a = p.A[h];
    if (tid < kQ) {
        const float dt = tid < len ? E::load(dl, (b * L + t0 + tid) * H + h) : 0.f;
        s_dt[tid] = dt;
        s_cum[tid] = dt * a;
        ssd_cumsum_wave(s_cum, tid);
    }
    __syncthreads();
    // M[t][s] = (C_t . B_s) exp(cum_t - cum_s) delta_s for s <= t, else 0
    for (int i = tid; i < kQ * kQ; i += 256) {
        const int t = i / kQ, s = i % kQ;
        float v = 0.f;
        if (s <= t) {
            float g = 0.f;
            for (int n = 0; n < N; ++n) g = fmaf(s_c[t][n], s_b[s][n], g);
            v = g * expf(s_cum[t] - s_cum[s]) * s_dt[s];
        }
        s_m[t][s] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
    __syncthreads();
    // Y_intra: wave w computes rows i0 .. i0+31, columns j0 .. j0+31; column
    // blocks past the rows are zero (causal) and skipped
    const int i0 = (wave >> 1) * 32, j0 = (wave & 1) * 32;
    ssd_f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int kh = lane >> 5;  // which 4 of the 8 k values of a step
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 8) {
        if (k0 >= i0 + 32) break;  // uniform per wave
        const ssd_bf16x4 av = *reinterpret_cast<const ssd_bf16x4*>(&s_m[i0 + (lane & 31)][k0 + 4 * kh]);
        const ssd_bf16x4 bv = *reinterpret_cast<const ssd_bf16x4*>(&s_xt[j0 + (lane & 31)][k0 + 4 * kh]);
        acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(av, bv, acc, 0, 0, 0);
    }
    // outputs: lane holds column j, rows i = i0 + 8 (r / 4) + 4 kh + r % 4
    const int j = j0 + (lane & 31);
    const float dsk = p.Dskip ? p.Dskip[h * kP + j] : 0.f;
    T* y = static_cast<T*>(p.y);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * kh + (r & 3);
        float inter = 0.f;
        for (int n = 0; n < N; ++n) inter = fmaf(s_c[i][n], s_h[n][j], inter);
        const float x = __uint_as_float(static_cast<uint32_t>(s_xt[j][i]) << 16);
        const float v = acc[r] + expf(s_cum[i]) * inter + dsk * x;
        if (i < len) E::store(y, (b * L + t0 + i) * D + h * kP + j, v);
    }
}

}  // namespace ssm
