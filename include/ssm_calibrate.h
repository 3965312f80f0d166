/*
 * ssm_calibrate.h -- measurement helpers exported by libssmscan.so.  They
 * are not part of the scan: one gives the HBM ceiling that the scan's
 * throughput is compared with, measured by a kernel of this library rather
 * than by a vendor copy routine; the other applies the scan's transcendental
 * policies element-wise so their accuracy can be measured.
 */
#ifndef SSM_CALIBRATE_H
#define SSM_CALIBRATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A read-dominant HBM stream shaped like the scan's traffic: it reads every
 * byte of `src` once and writes every byte of `dst` once, with
 * ratio = src_bytes / dst_bytes reads per write.  Each thread sums `ratio`
 * 16-byte chunks of src that lie dst_bytes apart (so every load instruction
 * of a wave reads 1 KiB of consecutive bytes) and stores the sum to dst.
 *
 *   src, dst     device pointers, 16-byte aligned, not overlapping
 *   src_bytes    ratio * dst_bytes with an integer ratio in [1, 64]
 *   dst_bytes    a positive multiple of 16
 *   nontemporal  1: loads and stores carry the non-temporal hint; 0: default policy
 *   clocks       device pointer to 2 uint64 values, or NULL: the shader-clock
 *                counter (s_memtime) and the 100 MHz real-time counter
 *                (s_memrealtime) elapsed over the first workgroup's run (the
 *                whole kernel: every workgroup is resident from the start), so
 *                clocks[0] / clocks[1] * 100 MHz is the sustained shader clock
 *   stream       hipStream_t (NULL = default stream)
 *
 * The contents of src are arbitrary (summed as fp32); dst receives the sums.
 * Enqueues one kernel; no host synchronisation.  Returns 0, 1 for an invalid
 * argument (checked before any HIP call) or 4 for a HIP launch error (the
 * status codes of ssm_scan.h).
 */
int ssm_calibrate_stream(const void *src, size_t src_bytes, void *dst, size_t dst_bytes, int32_t nontemporal,
                         uint64_t *clocks, void *stream);

/*
 * The scan kernel's own transcendental policies (csrc/device_math.h) applied
 * element-wise, for measuring their accuracy and bias against fp64: the same
 * inline functions the chunked kernel calls, so the figures describe what
 * the scan computes.  out[i] = f(x[i], y[i]) for i < n, with fn:
 *   0  exp(x * y) as exp(delta A): 2^(x * (y log2 e)) on the hardware exp2
 *   1  sin(x), 2  cos(x): hardware sin/cos on fract(x / 2 pi) (bf16-I/O path)
 *   3  sin(x), 4  cos(x): Cephes polynomials, valid for |x| <= pi/4 (fp32 path)
 *   5  sin(x), 6  cos(x): fp64 Cody-Waite reduction, then the polynomials (fp32 path)
 *   7  e^z - 1, 8  e^z, z = x * y, as the ZOH weight computes them
 * y is read only by fn 0, 7 and 8 (it may be NULL otherwise).
 *
 *   x, y, out    device pointers to n fp32 values (out does not overlap x, y)
 *   n            element count, 0 <= n < 2^31
 *   stream       hipStream_t (NULL = default stream)
 *
 * Enqueues one kernel (none for n = 0); no host synchronisation.  Returns 0,
 * 1 for an invalid argument (checked before any HIP call) or 4 for a HIP
 * launch error.
 */
int ssm_calibrate_device_math(int32_t fn, const float *x, const float *y, float *out, int64_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CALIBRATE_H */
