// device_math.h -- exp and sin/cos policies of the chunked scan kernel.
//
// exp(delta*A): both policies use v_exp_f32, which computes 2^x, as
// 2^(delta * (A*log2 e)) with A*log2 e formed once per lane.  Measured on
// gfx950 over the workloads' ranges of delta*A the hardware 2^x is unbiased
// (mean error below 0.04 ulp, max 0.8 ulp); the only bias is the rounding of
// log2 e (relative 1.3e-8 times |delta*A|), whose sum over a state's memory
// stays near 2e-7.
//
// sin/cos of theta:
//   Fast (bf16 I/O): v_sin_f32 / v_cos_f32, which take their argument in
//   revolutions, on fract(theta / 2 pi) (the hardware is specified on +-256
//   revolutions).  Measured: sin within ~1e-7 absolute, cos within 2.1 ulp
//   with a mean bias of -0.6 ulp; fine for bf16 outputs, not for fp32 ones
//   (the bias compounds over a slowly decaying state).
//   Accurate (fp32 I/O): the Cephes single-precision sin/cos polynomials
//   (S. L. Moshier, Cephes Mathematical Library, sinf.c / cosf.c
//   coefficients for |x| <= pi/4; measured <= 0.75 ulp and unbiased) when the
//   caller has established |theta| <= pi/4.  Otherwise theta is first
//   reduced to r = theta - k pi/2, |r| <= pi/4, in fp64 (Cody-Waite with a
//   two-part pi/2 and fused multiply-adds: exact to far below fp32 resolution
//   for |theta| < 2^50), and the quadrant k mod 4 maps the polynomials'
//   (sin r, cos r) to (sin, cos) of theta.
// ZOH needs both e^z and e^z - 1 (z = delta*A; weight (e^z - 1)/A): on
// |z| <= ln2/2 the degree-7 Taylor polynomial of e^z - 1 (truncation below
// 1.6e-8 relative; 1.5 ulp measured in fp32) and e^z = 1 + that, elsewhere the
// hardware e^z and e^z - 1, which has no cancellation there (|e^z - 1| > 0.29).
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;
constexpr float kPiOver4 = 0.78539816339744831f;

// sin/cos variants a pass can be instantiated with
enum SinCos : int { kSinCosHw = 0, kSinCosPoly = 1, kSinCosWide = 2 };

// Cephes polynomials, |x| <= pi/4
__device__ __forceinline__ void sin_cos_poly(float x, float* s, float* c) {
    const float z = x * x;
    *s = ((-1.9515295891e-4f * z + 8.3321608736e-3f) * z - 1.6666654611e-1f) * z * x + x;
    *c = ((2.443315711809948e-5f * z - 1.388731625493765e-3f) * z + 4.166664568298827e-2f) * z * z - 0.5f * z + 1.0f;
}

// A as stored per lane: pre-multiplied by log2(e).
__device__ __forceinline__ float prep_A(float a) { return a * kLog2e; }
// exp(delta * A) from delta and prep_A(A)
__device__ __forceinline__ float exp_dA(float delta, float a_prep) { return __builtin_amdgcn_exp2f(delta * a_prep); }

// sin/cos of an angle given in revolutions, |rev| < 256 (hardware units)
__device__ __forceinline__ void sin_cos_rev(float rev, float* s, float* c) {
    *s = __builtin_amdgcn_sinf(rev);
    *c = __builtin_amdgcn_cosf(rev);
}

// sin/cos of an fp64 angle: reduced to |r| <= pi/4 in fp64 (Cody-Waite, two-part
// pi/2, fused multiply-adds), then the polynomials and the quadrant map
__device__ __forceinline__ void sin_cos_wide(double t, float* s, float* c) {
    constexpr double kTwoOverPi = 0.63661977236758134308;
    constexpr double kPiOver2Hi = 1.5707963267948966;     // pi/2 rounded to double
    constexpr double kPiOver2Lo = 6.123233995736766e-17;  // pi/2 - kPiOver2Hi
    const double k = __builtin_rint(t * kTwoOverPi);
    const double r = __builtin_fma(-k, kPiOver2Lo, __builtin_fma(-k, kPiOver2Hi, t));
    float sr, cr;
    sin_cos_poly(static_cast<float>(r), &sr, &cr);
    const int q = static_cast<int>(static_cast<long long>(k) & 3);  // k finite here, else r is NaN
    const float ss = (q & 1) ? cr : sr, cc = (q & 1) ? sr : cr;
    *s = (q & 2) ? -ss : ss;
    *c = ((q + 1) & 2) ? -cc : cc;
}

// e^z and e^z - 1 from z and z*log2(e)
__device__ __forceinline__ void exp_expm1(float z, float z_log2e, float* ez, float* em1) {
    constexpr float kLn2Half = 0.34657359027997264f;
    float p = 1.0f / 5040.0f;
    p = p * z + 1.0f / 720.0f;
    p = p * z + 1.0f / 120.0f;
    p = p * z + 1.0f / 24.0f;
    p = p * z + 1.0f / 6.0f;
    p = p * z + 0.5f;
    p = p * z + 1.0f;
    p = p * z;  // e^z - 1 near 0
    const float e = __builtin_amdgcn_exp2f(z_log2e);
    const bool small = fabsf(z) <= kLn2Half;
    *em1 = small ? p : e - 1.0f;
    *ez = small ? 1.0f + p : e;
}

template <int SC>
__device__ __forceinline__ void sin_cos(float th, float* s, float* c) {
    if constexpr (SC == kSinCosHw) {
        const float r = __builtin_amdgcn_fractf(th * kInv2Pi);
        *s = __builtin_amdgcn_sinf(r);
        *c = __builtin_amdgcn_cosf(r);
    } else if constexpr (SC == kSinCosPoly) {  // |th| <= pi/4
        sin_cos_poly(th, s, c);
    } else {
        sin_cos_wide(static_cast<double>(th), s, c);
    }
}

}  // namespace ssm
