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
// Every term is a dense contraction and runs on the bf16 MFMA units
// (gfx950's v_mfma_f32_32x32x16_bf16, fp32 accumulation): C B^T (Q x N . N x Q), the
// intra-chunk product (Q x Q . Q x P), C H_in (Q x N . N x P) and the chunk
// state (N x Q . Q x P).  The operands are rounded to bf16 (u, B and C are
// bf16 already; the decay-weighted matrix, the weighted B and H_in are
// rounded); exp of the cumulative decays runs on the vector units.
//
// Three kernels (per batch row b and head h, chunks of Q = 64 steps, heads of
// P = 64 channels):
//   ssd_state_kernel  each chunk's local state contribution S_c (N x P) and
//                     its decay e_c = exp(cum_{Q-1}), all chunks in parallel;
//   ssd_pass_kernel   the states entering each chunk, H_in(c+1) = e_c H_in(c)
//                     + S_c, one thread per state element walking the chunks
//                     (the running state in fp32; S and H_in are kept in bf16,
//                     the precision the output products read H_in in);
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
    uint16_t* S;        // [B][H][nC][N][P]  chunk contributions, bf16 (workspace)
    float* E;           // [B][H][nC]        chunk decays (workspace)
    uint16_t* Hin;      // [B][H][nC][N][P]  state entering each chunk, bf16 (workspace)
    int64_t batch, seqlen, dim, dstate, heads, nchunks;
    int32_t bc_vec;     // N a multiple of 8 and B, C 16-byte aligned: rows move in 16-byte pieces
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

typedef short ssd_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 ssd_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ssd_f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t ssd_bf16(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float ssd_widen(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// One 32 x 32 block of A . B with K = 8 * ksteps on the bf16 MFMA units, both
// operands in LDS with k contiguous: a_rows[i][k] (rows i0 ..) and b_cols[j][k]
// (columns j0 ..).  Pairs of 8-wide k steps go to one 32x32x16 instruction,
// for which lane l supplies A[i0 + l % 32][k0 + 8 (l / 32) + 0..7] and
// B[k0 + 8 (l / 32) + 0..7][j0 + l % 32] (one 16-byte LDS read each); an odd
// last step uses the 32x32x8 form, lane l supplying 4 values at
// k0 + 4 (l / 32).  Both leave the 32 x 32 result spread as
// acc[r] = C[i0 + 8 (r / 4) + 4 (l / 32) + r % 4][j0 + l % 32].
template <int kStride>
__device__ __forceinline__ void ssd_mfma_block(const uint16_t (*a_rows)[kStride], const uint16_t (*b_cols)[kStride],
                                               int i0, int j0, int ksteps, int lane, ssd_f32x16& acc) {
    static_assert(kStride % 8 == 0, "16-byte operand rows");
    const int kh = lane >> 5;
    int ks = 0;
    for (; ks + 2 <= ksteps; ks += 2) {
        const int k0 = ks * 8 + 8 * kh;
        const ssd_bf16x8 av = *reinterpret_cast<const ssd_bf16x8*>(&a_rows[i0 + (lane & 31)][k0]);
        const ssd_bf16x8 bv = *reinterpret_cast<const ssd_bf16x8*>(&b_cols[j0 + (lane & 31)][k0]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    if (ks < ksteps) {
        const int k0 = ks * 8 + 4 * kh;
        const ssd_bf16x4 av = *reinterpret_cast<const ssd_bf16x4*>(&a_rows[i0 + (lane & 31)][k0]);
        const ssd_bf16x4 bv = *reinterpret_cast<const ssd_bf16x4*>(&b_cols[j0 + (lane & 31)][k0]);
        acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(av, bv, acc, 0, 0, 0);
    }
}

constexpr float kSsdLog2e = 1.4426950408889634f;

// row of element r of a lane's 32 x 32 accumulator block
__device__ __forceinline__ int ssd_acc_row(int i0, int lane, int r) {
    return i0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// NMAX: the largest N the instantiation handles (16 or 64); it sizes the LDS
// tiles, so small state sizes leave room for more resident workgroups.
// The 16-byte pieces of X (the head's 64 channels of a step are one 128-byte
// row) and of the B or C rows of a chunk (8 states each) that one thread
// loads, all issued before any is used so that a workgroup waits for memory
// once.  Rows past the sequence end read the chunk's last valid row instead
// (no branch around a load) and are zeroed when stored to LDS.
template <typename T>
__device__ __forceinline__ uint4 ssd_ld16(const T* p) {
    return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
__device__ __forceinline__ void ssd_load_x(const T* u, int64_t row0, int64_t D, int len, int tid,
                                           uint4 (&xv)[ssd::kQ * ssd::kP / 8 / 256]) {
#pragma unroll
    for (int q = 0; q < ssd::kQ * ssd::kP / 8 / 256; ++q) {
        const int i = tid + 256 * q, t = i / (ssd::kP / 8), p8 = (i % (ssd::kP / 8)) * 8;
        xv[q] = ssd_ld16(u + (row0 + (t < len ? t : len - 1)) * D + p8);
    }
}

// X transposed into LDS (rows p, columns t) from the pieces of ssd_load_x
__device__ __forceinline__ void ssd_store_xt(const uint4 (&xv)[ssd::kQ * ssd::kP / 8 / 256], int len, int tid,
                                             uint16_t (*s_xt)[ssd::kQ + ssd::kPad]) {
#pragma unroll
    for (int q = 0; q < ssd::kQ * ssd::kP / 8 / 256; ++q) {
        const int i = tid + 256 * q, t = i / (ssd::kP / 8), p8 = (i % (ssd::kP / 8)) * 8;
        const bool ok = t < len;
        const uint32_t w[4] = {ok ? xv[q].x : 0u, ok ? xv[q].y : 0u, ok ? xv[q].z : 0u, ok ? xv[q].w : 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s_xt[p8 + 2 * k][t] = static_cast<uint16_t>(w[k]);
            s_xt[p8 + 2 * k + 1][t] = static_cast<uint16_t>(w[k] >> 16);
        }
    }
}

// NMAX: the largest N the instantiation handles (16 or 64); it sizes the LDS
// tiles, so small state sizes leave room for more resident workgroups.
template <typename T, int NMAX>
__global__ void __launch_bounds__(256) ssd_state_kernel(SsdParams p) {
    using namespace ssd;
    using E = Elem<T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nC = p.nchunks, H = p.heads, L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t c = blockIdx.x % nC, bh = blockIdx.x / nC, b = bh / H, h = bh % H;
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    // S = (B o w)^T X as an (N x Q)(Q x P) product: rows n (padded to 64),
    // k = t contiguous in both operands
    constexpr int kRows = NMAX <= 32 ? 32 : 64;                  // n rows, padded to MFMA blocks
    __shared__ __align__(16) uint16_t s_bw[kRows][kQ + kPad];  // B[t][n] w_t, transposed
    __shared__ __align__(16) uint16_t s_xt[kP][kQ + kPad];     // X transposed
    __shared__ float s_cum[kQ], s_w[kQ];
    const T* u = static_cast<const T*>(p.u);
    const T* Bm = static_cast<const T*>(p.B);
    const T* dl = static_cast<const T*>(p.delta);
    // every global load first: X, B (16-byte pieces when bc_vec), delta
    uint4 xv[kQ * kP / 8 / 256];
    ssd_load_x<T>(u + h * kP, b * L + t0, D, len, tid, xv);
    constexpr int kBV = (kQ * NMAX / 8 + 255) / 256;  // B pieces per thread at N = NMAX
    const int nv = static_cast<int>(N / 8), pieces = kQ * nv;
    uint4 bv[kBV];
    if (p.bc_vec) {
#pragma unroll
        for (int q = 0; q < kBV; ++q) {
            const int i = tid + 256 * q < pieces ? tid + 256 * q : pieces - 1, t = i / nv, n8 = (i % nv) * 8;
            bv[q] = ssd_ld16(Bm + (b * L + t0 + (t < len ? t : len - 1)) * N + n8);
        }
    }
    const int tl = lane < len ? lane : len - 1;
    const float dt_raw = E::load(dl, (b * L + t0 + tl) * H + h);
    // cumulative decays in log2 units: exp(cum) = 2^(cum log2 e) on the hardware exp2
    const float a2 = p.A[h] * kSsdLog2e;
    if (tid < kQ) {
        const float dt = tid < len ? dt_raw : 0.f;
        s_cum[tid] = dt * a2;
        ssd_cumsum_wave(s_cum, tid);
        s_w[tid] = dt * __builtin_amdgcn_exp2f(s_cum[kQ - 1] - s_cum[tid]);  // exp(cum_{Q-1} - cum_t) delta_t
    }
    ssd_store_xt(xv, len, tid, s_xt);
    __syncthreads();
    const int nrows = N <= 32 ? 32 : kRows;
    if (p.bc_vec) {
        // rows n >= N of s_bw stay as they are: they only feed result rows n >= N, which are not stored
#pragma unroll
        for (int q = 0; q < kBV; ++q) {
            const int i = tid + 256 * q;
            if (i < pieces) {
                const int t = i / nv, n8 = (i % nv) * 8;
                const float w = t < len ? s_w[t] : 0.f;
                const uint32_t x[4] = {bv[q].x, bv[q].y, bv[q].z, bv[q].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s_bw[n8 + 2 * k][t] = ssd_bf16(bf16_lo(x[k]) * w);
                    s_bw[n8 + 2 * k + 1][t] = ssd_bf16(bf16_hi(x[k]) * w);
                }
            }
        }
    } else {
        for (int i = tid; i < nrows * kQ; i += 256) {
            const int n = i / kQ, t = i % kQ;
            const float v = (n < N && t < len) ? E::load(Bm, (b * L + t0 + t) * N + n) * s_w[t] : 0.f;
            s_bw[n][t] = ssd_bf16(v);
        }
    }
    __syncthreads();
    // wave w: rows n0 = 32 (w / 2) (if present), columns p0 = 32 (w % 2)
    const int n0 = 32 * (wave >> 1), p0 = 32 * (wave & 1);
    if (n0 < nrows) {
        ssd_f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        ssd_mfma_block<kQ + kPad>(s_bw, s_xt, n0, p0, kQ / 8, lane, acc);
        uint16_t* S = p.S + (bh * nC + c) * N * kP;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int n = ssd_acc_row(n0, lane, r);
            if (n < N) S[n * kP + p0 + (lane & 31)] = ssd_bf16(acc[r]);
        }
    }
    if (tid == 0) p.E[bh * nC + c] = __builtin_amdgcn_exp2f(s_cum[kQ - 1]);
}

__global__ void __launch_bounds__(256) ssd_pass_kernel(SsdParams p) {
    using namespace ssd;
    const int64_t nC = p.nchunks, H = p.heads, N = p.dstate;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // (b, h, n, pp)
    if (i >= p.batch * H * N * kP) return;
    const int64_t bh = i / (N * kP), np = i % (N * kP);
    const uint16_t* S = p.S + bh * nC * N * kP + np;
    uint16_t* Hin = p.Hin + bh * nC * N * kP + np;
    const float* E = p.E + bh * nC;
    float st = 0.f;
    int64_t c = 0;
    // eight chunks' loads at a time, then the dependent chain over them
    for (; c + 8 <= nC; c += 8) {
        float s[8], e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s[k] = ssd_widen(S[(c + k) * N * kP]);
            e[k] = E[c + k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            Hin[(c + k) * N * kP] = ssd_bf16(st);
            st = fmaf(e[k], st, s[k]);
        }
    }
    for (; c < nC; ++c) {
        Hin[c * N * kP] = ssd_bf16(st);
        st = fmaf(E[c], st, ssd_widen(S[c * N * kP]));
    }
    if (p.h_last) {
        const int64_t b = bh / H, h = bh % H, n = np / kP, pp = np % kP;
        p.h_last[(b * p.dim + h * kP + pp) * N + n] = st;
    }
}

// Six workgroups per CU: LDS of about 19 KB (N <= 16) and at most 80 VGPRs.
template <typename T, int NMAX>
__global__ void __launch_bounds__(256, 6) ssd_out_kernel(SsdParams p) {
    using namespace ssd;
    using E = Elem<T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nC = p.nchunks, H = p.heads, L = p.seqlen, D = p.dim, N = p.dstate;
    const int64_t c = blockIdx.x % nC, bh = blockIdx.x / nC, b = bh / H, h = bh % H;
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    const int npad = static_cast<int>((N + 7) / 8 * 8);  // K of the products over n
    // bf16 MFMA operands, k contiguous: C and B rows (k = n), H_in transposed
    // (rows p, k = n), X transposed (rows p, k = s), M (rows t, k = s).  M
    // (and later the output tile) takes the space of C, B and H_in, which are
    // dead once every wave has formed its G and C H_in blocks.
    static_assert(kP == kQ, "H_in rows share the C and B tiles' shape");
    constexpr int kRowN = NMAX + kPad, kRowQ = kQ + kPad;
    constexpr int kUnion = 3 * kQ * kRowN > kQ * kRowQ ? 3 * kQ * kRowN : kQ * kRowQ;
    __shared__ __align__(16) uint16_t s_u[kUnion];
    __shared__ __align__(16) uint16_t s_xt[kP][kRowQ];
    __shared__ float s_cum[kQ], s_dt[kQ];
    uint16_t (*s_c)[kRowN] = reinterpret_cast<uint16_t (*)[kRowN]>(s_u);
    uint16_t (*s_b)[kRowN] = reinterpret_cast<uint16_t (*)[kRowN]>(s_u + kQ * kRowN);
    uint16_t (*s_ht)[kRowN] = reinterpret_cast<uint16_t (*)[kRowN]>(s_u + 2 * kQ * kRowN);
    uint16_t (*s_m)[kRowQ] = reinterpret_cast<uint16_t (*)[kRowQ]>(s_u);
    const T* u = static_cast<const T*>(p.u);
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);
    const T* dl = static_cast<const T*>(p.delta);
    const uint16_t* Hin = p.Hin + (bh * nC + c) * N * kP;
    // every global load first (one wait for memory): X; B, C and H_in in
    // 16-byte pieces when bc_vec; delta; D of this lane's output column
    uint4 xv[kQ * kP / 8 / 256];
    ssd_load_x<T>(u + h * kP, b * L + t0, D, len, tid, xv);
    constexpr int kBV = (2 * kQ * NMAX / 8 + 255) / 256;  // B and C pieces per thread at N = NMAX
    constexpr int kHV = (NMAX * kP / 8 + 255) / 256;      // H_in pieces per thread at N = NMAX
    const int nv = static_cast<int>(N / 8), bpieces = kQ * nv, hpieces = static_cast<int>(N) * (kP / 8);
    uint4 bcv[kBV], hv[kHV];
    if (p.bc_vec) {
#pragma unroll
        for (int q = 0; q < kBV; ++q) {
            int i = tid + 256 * q < 2 * bpieces ? tid + 256 * q : 2 * bpieces - 1;
            const T* src = i < bpieces ? Bm : Cm;
            i = i < bpieces ? i : i - bpieces;
            const int t = i / nv, n8 = (i % nv) * 8;
            bcv[q] = ssd_ld16(src + (b * L + t0 + (t < len ? t : len - 1)) * N + n8);
        }
#pragma unroll
        for (int q = 0; q < kHV; ++q) {
            const int i = tid + 256 * q < hpieces ? tid + 256 * q : hpieces - 1;
            hv[q] = ssd_ld16(Hin + i * 8);
        }
    }
    const int tl = lane < len ? lane : len - 1;
    const float dt_raw = E::load(dl, (b * L + t0 + tl) * H + h);
    const int j = 32 * (wave & 1) + (lane & 31);  // this lane's output column
    const float* dsp = p.Dskip ? p.Dskip + h * kP + j : p.A;
    const float dsv = *dsp;
    const float dsk = p.Dskip ? dsv : 0.f;
    const float a2 = p.A[h] * kSsdLog2e;  // cumulative decays in log2 units
    if (tid < kQ) {
        const float dt = tid < len ? dt_raw : 0.f;
        s_dt[tid] = dt;
        s_cum[tid] = dt * a2;
        ssd_cumsum_wave(s_cum, tid);
    }
    ssd_store_xt(xv, len, tid, s_xt);
    if (p.bc_vec) {
#pragma unroll
        for (int q = 0; q < kBV; ++q) {
            int i = tid + 256 * q;
            if (i < 2 * bpieces) {
                uint16_t (*dst)[kRowN] = i < bpieces ? s_b : s_c;
                i = i < bpieces ? i : i - bpieces;
                const int t = i / nv, n8 = (i % nv) * 8;
                *reinterpret_cast<uint4*>(&dst[t][n8]) = t < len ? bcv[q] : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int q = 0; q < kHV; ++q) {
            const int i = tid + 256 * q;
            if (i < hpieces) {
                const int n = i / (kP / 8), pp8 = (i % (kP / 8)) * 8;
                const uint32_t x[4] = {hv[q].x, hv[q].y, hv[q].z, hv[q].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s_ht[pp8 + 2 * k][n] = static_cast<uint16_t>(x[k]);
                    s_ht[pp8 + 2 * k + 1][n] = static_cast<uint16_t>(x[k] >> 16);
                }
            }
        }
    } else {
        for (int i = tid; i < kQ * npad; i += 256) {
            const int t = i / npad, n = i % npad;
            const bool ok = t < len && n < N;
            s_b[t][n] = ok ? ssd_bf16(E::load(Bm, (b * L + t0 + t) * N + n)) : uint16_t(0);
            s_c[t][n] = ok ? ssd_bf16(E::load(Cm, (b * L + t0 + t) * N + n)) : uint16_t(0);
        }
        for (int i = tid; i < npad * kP; i += 256) {
            const int n = i / kP, pp = i % kP;
            s_ht[pp][n] = n < N ? Hin[n * kP + pp] : uint16_t(0);
        }
    }
    __syncthreads();
    // wave w: G = C B^T block (rows t 32 (w / 2), columns s 32 (w % 2); the
    // block above the diagonal is never read) and the same block of C H_in,
    // then, once C, B and H_in are dead, M = G o exp(cum_t - cum_s) o delta_s
    // (zero above the diagonal) over their space
    const int i0 = 32 * (wave >> 1), j0 = 32 * (wave & 1);
    ssd_f32x16 g, acc, inter;
#pragma unroll
    for (int r = 0; r < 16; ++r) g[r] = acc[r] = inter[r] = 0.f;
    if (j0 <= i0) ssd_mfma_block<kRowN>(s_c, s_b, i0, j0, npad / 8, lane, g);
    ssd_mfma_block<kRowN>(s_c, s_ht, i0, j0, npad / 8, lane, inter);
    __syncthreads();
    if (j0 <= i0) {
        const int sc = j0 + (lane & 31);
        const float cs = s_cum[sc], ds = s_dt[sc];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = ssd_acc_row(i0, lane, r);
            s_m[t][sc] = ssd_bf16(sc <= t ? g[r] * __builtin_amdgcn_exp2f(s_cum[t] - cs) * ds : 0.f);
        }
    }
    __syncthreads();
    // Y = M X + diag(exp(cum)) C H_in: wave w computes rows i0, columns j0
    ssd_mfma_block<kRowQ>(s_m, s_xt, i0, j0, (i0 + 32) / 8, lane, acc);  // causal: k < i0 + 32
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = ssd_acc_row(i0, lane, r);
        const float x = __uint_as_float(static_cast<uint32_t>(s_xt[j][i]) << 16);
        v[r] = acc[r] + __builtin_amdgcn_exp2f(s_cum[i]) * inter[r] + dsk * x;
    }
    // the output tile goes through LDS (rows t, columns p; M's space, free once
    // every wave has finished its products) and out as 16-byte row pieces
    __syncthreads();
    uint16_t (*s_y)[kRowQ] = s_m;
#pragma unroll
    for (int r = 0; r < 16; ++r) s_y[ssd_acc_row(i0, lane, r)][j] = ssd_bf16(v[r]);
    __syncthreads();
    T* y = static_cast<T*>(p.y) + h * kP;
    for (int i = tid; i < kQ * kP / 8; i += 256) {
        const int t = i / (kP / 8), p8 = (i % (kP / 8)) * 8;
        if (t < len)
            *reinterpret_cast<uint4*>(y + (b * L + t0 + t) * D + p8) = *reinterpret_cast<const uint4*>(&s_y[t][p8]);
    }
}

}  // namespace ssm
