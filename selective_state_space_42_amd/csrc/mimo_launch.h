// mimo_launch.h -- parameters and launchers of the MIMO scan kernels
// (kernel_mimo.h), shared by the host code that validates the C ABI and the
// translation unit that holds the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct MimoParams {
    const void* u;       // [B][L][D][R]
    const void* delta;   // [B][L][D]
    const float* A;      // [D][N]
    const void* B;       // [B][L][N][R] or [B][L][N][R][2]
    const void* C;       // same layout as B
    const float* Dskip;  // [D] or NULL
    const void* theta;   // [B][L][D][N] or NULL
    const void* lambda;  // [B][L][D] (trapezoid)
    const float* h0;     // [B][D][N] or [B][D][N][2], or NULL
    const float* q0;     // trapezoid: q_{-1}, layout of h0, or NULL
    void* y;             // [B][L][D][R]
    float* h_last;       // layout of h0, or NULL
    float* q_last;       // trapezoid: q_{L-1}, layout of h0, or NULL
    float* carry;        // per chunk c < nchunks - 1 and (b, d, n): (P, h) complex (4 floats) or real (2)
    int64_t batch, seqlen, dim, dstate;
    int64_t chunk;  // steps per time chunk
    int32_t nchunks;
    int32_t lpc;  // lanes per channel: power of two, 2 lpc >= dstate, lpc >= R, lpc <= 32
};

struct MimoStepParams {
    const void* u;       // [B][D][R]
    const void* delta;   // [B][D]
    const float* A;      // [D][N]
    const void* B;       // [B][N][R] or [B][N][R][2]
    const void* C;       // same layout as B
    const float* Dskip;  // [D] or NULL
    const void* theta;   // [B][D][N] or NULL
    const void* lambda;  // [B][D] (trapezoid)
    const void* u_prev;  // trapezoid: [B][D][R] of the previous step, or NULL (no previous step)
    const void* B_prev;  // trapezoid: like B, of the previous step (NULL with u_prev)
    float* h;            // [B][D][N] or [B][D][N][2], read and overwritten
    void* y;             // [B][D][R]
    int64_t batch, dim, dstate;
    int32_t lpc;    // as for MimoParams
    int32_t pairs;  // N even and h aligned to a lane's two states: one vector load and store each
};

// Enqueue the MIMO scan (time-chunk kernels, carry, output) or one decode
// step on `s`.  The caller has validated every argument; rank is 1, 2, 4 or 8.
hipError_t launch_mimo_scan(const MimoParams& p, bool bf16, int disc, bool cplx, int rank, hipStream_t s);
hipError_t launch_mimo_step(const MimoStepParams& p, bool bf16, int disc, bool cplx, int rank, hipStream_t s);

}  // namespace ssm
