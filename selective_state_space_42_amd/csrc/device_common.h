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
    // elements i, i+1 as one 8-byte load (i even, p 8-byte aligned)
    static __device__ __forceinline__ void load_pair(const float* p, int64_t i, float* lo, float* hi) {
        const float2 v = *reinterpret_cast<const float2*>(p + i);
        *lo = v.x;
        *hi = v.y;
    }
};

template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) {
        p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
    // elements i, i+1 as one 4-byte load (i even, p 4-byte aligned)
    static __device__ __forceinline__ void load_pair(const uint16_t* p, int64_t i, float* lo, float* hi) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
        *lo = __uint_as_float(w << 16);
        *hi = __uint_as_float(w & 0xffff0000u);
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

// ---- buffer resources: hardware range checking (raw buffers, stride 0):
// loads at a byte offset >= num_records return 0, stores there are dropped.
// The range check applies to the per-lane (VGPR) offset, so every offset is
// passed there.  Resource word 3 (0x00020000: 32-bit data format) is the
// raw-buffer setting for gfx9-family GPUs.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOutOfRange = 0x7fffff00u;  // a lane offset beyond any window

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

template <typename T>
struct Buf;

template <>
struct Buf<float> {
    static constexpr uint32_t kSize = 4;
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    static __device__ __forceinline__ void load_pair(rsrc_t r, uint32_t off, float* lo, float* hi) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        *lo = __builtin_bit_cast(float, static_cast<uint32_t>(v[0]));
        *hi = __builtin_bit_cast(float, static_cast<uint32_t>(v[1]));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    }
    // the stored bits, undecoded (decode with widen())
    static __device__ __forceinline__ uint32_t load_raw(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw); }
};

template <>
struct Buf<uint16_t> {
    static constexpr uint32_t kSize = 2;
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
    }
    static __device__ __forceinline__ void load_pair(rsrc_t r, uint32_t off, float* lo, float* hi) {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        *lo = __uint_as_float(w << 16);
        *hi = __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, off, 0, 0);
    }
    // the stored bits, undecoded (decode with widen())
    static __device__ __forceinline__ uint32_t load_raw(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
    static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw << 16); }
};

// An empty asm that claims to modify `v`: code depending on a prefetched
// value cannot be scheduled above this point, so the wait for the load lands
// here (where it has long completed) and not next to the load.
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

}  // namespace ssm
