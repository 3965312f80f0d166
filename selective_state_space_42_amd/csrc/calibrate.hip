// calibrate.hip -- the read-dominant HBM stream of include/ssm_calibrate.h.
//
// Thread i of the grid-stride loop sums chunks i, i + n, ..., i + (ratio-1) n
// of src (16-byte chunks, n = dst chunks) and writes chunk i of dst, so a
// wave's load reads 1 KiB of consecutive memory and every byte of src and dst
// moves once.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_math.h"
#include "ssm_calibrate.h"

namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ f4v load16(const f4v* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__global__ void __launch_bounds__(256) stream_kernel(const f4v* __restrict__ src, f4v* __restrict__ dst, uint64_t n,
                                                     int ratio, uint64_t* clocks) {
    const bool timer = clocks && blockIdx.x == 0 && threadIdx.x == 0;
    uint64_t t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        f4v acc = {0.f, 0.f, 0.f, 0.f};
        int m = 0;
        // four independent loads in flight per thread
        for (; m + 4 <= ratio; m += 4) {
            const f4v a = load16<NT>(src + i + (m + 0) * n);
            const f4v b = load16<NT>(src + i + (m + 1) * n);
            const f4v c = load16<NT>(src + i + (m + 2) * n);
            const f4v d = load16<NT>(src + i + (m + 3) * n);
            acc += (a + b) + (c + d);
        }
        for (; m < ratio; ++m) acc += load16<NT>(src + i + m * n);
        if constexpr (NT)
            __builtin_nontemporal_store(acc, dst + i);
        else
            dst[i] = acc;
    }
    if (clocks && blockIdx.x == 0) {  // uniform over the workgroup
        __syncthreads();                  // its last loads have been consumed
        if (timer) {
            clocks[0] = __builtin_amdgcn_s_memtime() - t0;
            clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
        }
    }
}

// out[i] = f(x[i], y[i]) by the scan's own policies (see the header)
__global__ void __launch_bounds__(256) math_eval_kernel(int fn, const float* __restrict__ x,
                                                        const float* __restrict__ y, float* __restrict__ out,
                                                        int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float a = x[i];
    const float b = (fn == 0 || fn >= 7) ? y[i] : 0.f;
    float s = 0.f, c = 0.f, r = 0.f;
    switch (fn) {
        case 0:
            r = ssm::exp_dA(a, ssm::prep_A(b));
            break;
        case 1:
        case 2:
            ssm::sin_cos_rev(__builtin_amdgcn_fractf(__builtin_fmaf(a, ssm::kInv2Pi, 0.f)), &s, &c);
            r = fn == 1 ? s : c;
            break;
        case 3:
        case 4:
            ssm::sin_cos_poly(a, &s, &c);
            r = fn == 3 ? s : c;
            break;
        case 5:
        case 6:
            ssm::sin_cos_wide(static_cast<double>(a), &s, &c);
            r = fn == 5 ? s : c;
            break;
        default: {
            float ez, em1;
            ssm::exp_expm1(a * b, a * ssm::prep_A(b), &ez, &em1);
            r = fn == 7 ? em1 : ez;
        }
    }
    out[i] = r;
}

}  // namespace

extern "C" int ssm_calibrate_device_math(int32_t fn, const float* x, const float* y, float* out, int64_t n,
                                    void* stream) {
    if (fn < 0 || fn > 8 || n < 0 || n >= (int64_t(1) << 31)) return 1;
    if (n == 0) return 0;
    const bool needs_y = fn == 0 || fn >= 7;
    if (!x || !out || (needs_y && !y)) return 1;
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + static_cast<uintptr_t>(n) * 4;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), x1 = x0 + static_cast<uintptr_t>(n) * 4;
    if (o0 < x1 && x0 < o1) return 1;
    if (needs_y) {
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + static_cast<uintptr_t>(n) * 4;
        if (o0 < y1 && y0 < o1) return 1;
    }
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(math_eval_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), fn, x, y, out, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int ssm_calibrate_stream(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                    int32_t nontemporal, uint64_t* clocks, void* stream) {
    if (!src || !dst || dst_bytes == 0 || dst_bytes % 16 != 0 || src_bytes % dst_bytes != 0) return 1;
    const size_t ratio = src_bytes / dst_bytes;
    if (ratio < 1 || ratio > 64) return 1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return 1;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return 1;  // overlapping
    if (nontemporal != 0 && nontemporal != 1) return 1;
    if (clocks && reinterpret_cast<uintptr_t>(clocks) % 8 != 0) return 1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 4;
    const uint64_t n = dst_bytes / 16;
    uint64_t blocks = static_cast<uint64_t>(cus) * 16;  // 16 workgroups of 4 waves per CU
    if (blocks > (n + 255) / 256) blocks = (n + 255) / 256;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f4v* sp = static_cast<const f4v*>(src);
    f4v* dp = static_cast<f4v*>(dst);
    if (nontemporal)
        hipLaunchKernelGGL(stream_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, sp, dp, n,
                           static_cast<int>(ratio), clocks);
    else
        hipLaunchKernelGGL(stream_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, sp, dp, n,
                           static_cast<int>(ratio), clocks);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
