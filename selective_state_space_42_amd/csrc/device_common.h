// device_common.h -- element I/O and small helpers shared by the scan kernels.
//
// Storage types: fp32 is `float`; bf16 is carried as its 16-bit pattern
// (`uint16_t`).  Widening bf16 -> fp32 is exact (the pattern moves to the top
// half of the fp32 word); narrowing fp32 -> bf16 rounds to nearest-even
// (gfx950's v_cvt_pk_bf16_f32 via the __bf16 conversion).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

enum Disc : int { kZOH = 0, kEuler = 1, kTrap = 2 };

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};

template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) {
        p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
};

// Both halves of a 32-bit word holding two bf16 values, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values rounded to nearest-even into one word of two bf16 (lo, hi).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi))) << 16);
}

}  // namespace ssm
