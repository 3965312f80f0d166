// device_math.h -- exp and sin/cos policies of the chunked scan kernel.
//
// Fast (bf16 I/O): the hardware transcendentals.  v_exp_f32 computes 2^x, so
// exp(delta*A) is evaluated as 2^(delta * (A*log2 e)) with A*log2 e formed
// once per lane; v_sin_f32 / v_cos_f32 take their argument in revolutions, so
// theta is scaled by 1/(2 pi) and reduced to [0, 1) with v_fract_f32 (the
// hardware is only specified on +-256 revolutions).  Measured on gfx950 over
// the workloads' ranges: 2^x within 0.8 ulp, sin within ~1e-7 absolute, cos
// within 2.1 ulp with a mean bias of -0.6 ulp; fine for bf16 outputs, not for
// fp32 ones.
//
// Accurate (fp32 I/O): the device library's expf / expm1f (unbiased, < 1 ulp
// in the measurement above) and, when every lane's |theta| <= pi/4, the
// Cephes single-precision sin/cos polynomials (S. L. Moshier, Cephes
// Mathematical Library, sinf.c / cosf.c coefficients for |x| <= pi/4; measured
// <= 0.75 ulp and unbiased); otherwise the device library's sincosf.
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;
constexpr float kPiOver4 = 0.78539816339744831f;

struct FastMath {
    // A as stored per lane: pre-multiplied by log2(e).
    static __device__ __forceinline__ float prep_A(float a) { return a * kLog2e; }
    // exp(delta * A) from delta and prep_A(A)
    static __device__ __forceinline__ float exp_dA(float delta, float a_prep) {
        return __builtin_amdgcn_exp2f(delta * a_prep);
    }
    static __device__ __forceinline__ void sincos(float th, float* s, float* c) {
        const float r = __builtin_amdgcn_fractf(th * kInv2Pi);
        *s = __builtin_amdgcn_sinf(r);
        *c = __builtin_amdgcn_cosf(r);
    }
};

struct AccurateMath {
    static __device__ __forceinline__ float prep_A(float a) { return a; }
    static __device__ __forceinline__ float exp_dA(float delta, float a) { return expf(delta * a); }
    static __device__ __forceinline__ void sincos(float th, float* s, float* c) {
        if (__any(!(fabsf(th) <= kPiOver4))) {  // any lane out of range (or NaN)
            sincosf(th, s, c);
        } else {
            const float z = th * th;
            *s = ((-1.9515295891e-4f * z + 8.3321608736e-3f) * z - 1.6666654611e-1f) * z * th + th;
            *c = ((2.443315711809948e-5f * z - 1.388731625493765e-3f) * z + 4.166664568298827e-2f) * z * z -
                 0.5f * z + 1.0f;
        }
    }
};

// ZOH input weight expm1(delta*A)/A, with its limit delta at A = 0.
// `inv_a` is 1/A (any value when A = 0).
__device__ __forceinline__ float zoh_gamma(float delta, float a, float inv_a) {
    return (a != 0.0f) ? expm1f(delta * a) * inv_a : delta;
}

}  // namespace ssm
