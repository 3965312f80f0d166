// ssm_scan.hip -- host side of libssmscan.so: argument validation, kernel
// choice, workspace sizing and launches behind the C ABI of include/ssm_scan.h.
//
// Validation happens before any HIP call, so every error path can be
// exercised without a GPU.  The library allocates nothing and never
// synchronises the host; all work is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssm_scan.h"
#include "device_common.h"
#include "kernel_sequential.h"
#include "kernel_sweep.h"
#include "kernel_chunked.h"
#include "kernel_step.h"
#include "kernel_backward.h"
#include "kernel_ssd.h"
#include "mimo_launch.h"

// The fixed scratch buffer of ssm_scan_fwd_noalloc: one copy per GPU, held
// from the loading of this code object on that GPU until the process ends.
// In host code `scratch` only names the symbol; its device address (a
// different one on each GPU) comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SSM_SCAN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

// Device address of `scratch` on each GPU, looked up once per device with
// that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr after storing the
// failing HIP error (or when the device index is out of range).
void* scratch_for_current_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        g_last_hip_error = static_cast<int>(hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            g_last_hip_error = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return SSM_OK;
    g_last_hip_error = static_cast<int>(e);
    return SSM_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int next_pow2(int64_t v) {
    int r = 1;
    while (r < v) r <<= 1;
    return r;
}

// Shape and mode checks shared by ssm_scan_workspace_bytes and ssm_scan_fwd.
int check_desc(const ssm_scan_desc_t* d) {
    if (!d) return SSM_ERR_INVALID_ARGUMENT;
    if (d->batch < 1 || d->seqlen < 1 || d->dim < 1 || d->dstate < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (d->io_dtype != SSM_DTYPE_F32 && d->io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
    if (d->disc < SSM_DISC_ZOH || d->disc > SSM_DISC_EXP_TRAPEZOIDAL) return SSM_ERR_UNSUPPORTED;
    if (d->is_complex != 0 && d->is_complex != 1) return SSM_ERR_UNSUPPORTED;
    if (d->algo < SSM_ALGO_AUTO || d->algo > SSM_ALGO_SWEEP) return SSM_ERR_UNSUPPORTED;
    if (d->is_complex && d->disc == SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d->dstate > 64) return SSM_ERR_UNSUPPORTED;
    // B*L*D*N*2 complex words of 4 bytes must fit an int64 byte offset.
    int64_t v = d->batch, r;
    if (__builtin_mul_overflow(v, d->seqlen, &r)) return SSM_ERR_INVALID_ARGUMENT;
    if (__builtin_mul_overflow(r, d->dim, &r)) return SSM_ERR_INVALID_ARGUMENT;
    if (__builtin_mul_overflow(r, d->dstate, &r)) return SSM_ERR_INVALID_ARGUMENT;
    if (__builtin_mul_overflow(r, int64_t(8), &r)) return SSM_ERR_INVALID_ARGUMENT;
    return SSM_OK;
}

// Kernel family for a valid descriptor.
int choose_algo(const ssm_scan_desc_t* d) {
    if (d->algo != SSM_ALGO_AUTO) return d->algo;
    if (d->dstate > ssm::kChunkLanes) return SSM_ALGO_SEQUENTIAL;
    if (ssm::sweep_preferred(d->batch, d->seqlen, d->dim, d->is_complex != 0, d->disc == SSM_DISC_EXP_TRAPEZOIDAL) &&
        ssm::sweep_offsets_fit(d->dim, d->dstate, d->io_dtype == SSM_DTYPE_F32 ? 4 : 2))
        return SSM_ALGO_SWEEP;
    return ssm::chunked_preferred(d->batch, d->seqlen, d->dim) ? SSM_ALGO_CHUNKED : SSM_ALGO_SEQUENTIAL;
}

// Shapes the lane sweep cannot take (explicit SSM_ALGO_SWEEP).
bool sweep_unsupported(const ssm_scan_desc_t* d) {
    return d->dstate > ssm::sweep::kLPC ||
           !ssm::sweep_offsets_fit(d->dim, d->dstate, d->io_dtype == SSM_DTYPE_F32 ? 4 : 2) ||
           (ssm::sweep_waves(d->batch, d->dim) + ssm::sweep::kWaves - 1) / ssm::sweep::kWaves > INT32_MAX;
}

template <typename T, int DISC, int WAVES>
void launch_sweep_c(const ssm::SweepParams& p, bool pairs, int64_t waves, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((waves + WAVES - 1) / WAVES)), block(WAVES * 64);
    if (pairs)
        hipLaunchKernelGGL((ssm::sweep_scan_kernel<T, DISC, true, true, WAVES>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((ssm::sweep_scan_kernel<T, DISC, true, false, WAVES>), grid, block, 0, s, p);
}
template <typename T, int DISC>
void launch_sweep_k(const ssm::SweepParams& p, bool pairs, int64_t waves, int wg_waves, hipStream_t s) {
    if (wg_waves == 16)
        launch_sweep_c<T, DISC, 16>(p, pairs, waves, s);
    else if (wg_waves == 8)
        launch_sweep_c<T, DISC, 8>(p, pairs, waves, s);
    else
        launch_sweep_c<T, DISC, ssm::sweep::kWaves>(p, pairs, waves, s);
}

// pairs: complex B and C aligned to whole (re, im) entries
template <typename T>
int launch_sweep(const ssm_scan_desc_t* d, const ssm::SweepParams& p, bool pairs, hipStream_t s) {
    const int64_t waves = ssm::sweep_waves(d->batch, d->dim);
    const int64_t blocks = (waves + ssm::sweep::kWaves - 1) / ssm::sweep::kWaves;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (d->is_complex) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_status(e);
        const int wg = ssm::sweep_wg_waves(waves, true, cus);
        if (d->disc == SSM_DISC_EXP_EULER)
            launch_sweep_k<T, ssm::kEuler>(p, pairs, waves, wg, s);
        else
            launch_sweep_k<T, ssm::kTrap>(p, pairs, waves, wg, s);
    } else {
        if (d->disc == SSM_DISC_ZOH)
            hipLaunchKernelGGL((ssm::sweep_scan_kernel<T, ssm::kZOH, false, false, ssm::sweep::kWaves>), grid,
                               dim3(ssm::sweep::kWaves * 64), 0, s, p);
        else if (d->disc == SSM_DISC_EXP_EULER)
            hipLaunchKernelGGL((ssm::sweep_scan_kernel<T, ssm::kEuler, false, false, ssm::sweep::kWaves>), grid,
                               dim3(ssm::sweep::kWaves * 64), 0, s, p);
        else
            hipLaunchKernelGGL((ssm::sweep_scan_kernel<T, ssm::kTrap, false, false, ssm::sweep::kWaves>), grid,
                               dim3(ssm::sweep::kWaves * 64), 0, s, p);
    }
    return hip_status(hipGetLastError());
}

template <typename T>
int launch_sequential(const ssm_scan_desc_t* d, const ssm::SeqParams& p, hipStream_t s) {
    const int64_t waves = (d->batch * d->dim + (64 / p.lpc) - 1) / (64 / p.lpc);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (d->is_complex) {
        if (d->disc == SSM_DISC_EXP_EULER)
            hipLaunchKernelGGL((ssm::scan_sequential_kernel<T, ssm::kEuler, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((ssm::scan_sequential_kernel<T, ssm::kTrap, true>), grid, block, 0, s, p);
    } else {
        if (d->disc == SSM_DISC_ZOH)
            hipLaunchKernelGGL((ssm::scan_sequential_kernel<T, ssm::kZOH, false>), grid, block, 0, s, p);
        else if (d->disc == SSM_DISC_EXP_EULER)
            hipLaunchKernelGGL((ssm::scan_sequential_kernel<T, ssm::kEuler, false>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((ssm::scan_sequential_kernel<T, ssm::kTrap, false>), grid, block, 0, s, p);
    }
    return hip_status(hipGetLastError());
}

template <typename T, bool PAIRS>
int launch_step_k(const ssm_scan_desc_t* d, const ssm::StepParams& p, hipStream_t s) {
    const int64_t waves = (d->batch * d->dim + (64 / p.lpc) - 1) / (64 / p.lpc);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    const bool th = p.theta != nullptr;
    if (d->is_complex) {
        if (d->disc == SSM_DISC_EXP_EULER) {
            if (th)
                hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kEuler, true, PAIRS, true>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kEuler, true, PAIRS, false>), grid, block, 0, s, p);
        } else {
            if (th)
                hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kTrap, true, PAIRS, true>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kTrap, true, PAIRS, false>), grid, block, 0, s, p);
        }
    } else {
        if (d->disc == SSM_DISC_ZOH)
            hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kZOH, false, PAIRS, false>), grid, block, 0, s, p);
        else if (d->disc == SSM_DISC_EXP_EULER)
            hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kEuler, false, PAIRS, false>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((ssm::scan_step_kernel<T, ssm::kTrap, false, PAIRS, false>), grid, block, 0, s, p);
    }
    return hip_status(hipGetLastError());
}

// The paired step kernel reads each lane's two states with one vector load
// per array: N even and every array aligned to a pair of its elements.
template <typename T>
int launch_step(const ssm_scan_desc_t* d, const ssm::StepParams& p, hipStream_t s) {
    const size_t es = sizeof(T), cw = d->is_complex ? 2 : 1;
    const bool pairs = d->dstate % 2 == 0 && aligned(p.h, 8 * cw) && aligned(p.A, 8) &&
                       aligned(p.B, 2 * cw * es) && aligned(p.C, 2 * cw * es) &&
                       (!p.B_prev || aligned(p.B_prev, 2 * cw * es)) && (!p.theta || aligned(p.theta, 2 * es));
    return pairs ? launch_step_k<T, true>(d, p, s) : launch_step_k<T, false>(d, p, s);
}

// grid: one copy of the channel waves (the checkpoint sweep) and one per time
// chunk (the adjoint and reverse sweeps)
template <typename T, int DISC, bool CPLX, int LPC>
void launch_bwd_kernels(const ssm::BwdParams& p, dim3 grid, dim3 chunk_grid, hipStream_t s) {
    hipLaunchKernelGGL((ssm::bwd_ckpt_kernel<T, DISC, CPLX, LPC>), grid, dim3(256), 0, s, p);
    if (p.nchunks > 1) {
        hipLaunchKernelGGL((ssm::bwd_adj_kernel<T, DISC, CPLX, LPC>), chunk_grid, dim3(256), 0, s, p);
        const int64_t bdn = p.batch * p.dim * p.dstate;
        hipLaunchKernelGGL((ssm::bwd_adj_carry_kernel<CPLX>), dim3(static_cast<unsigned>((bdn + 255) / 256)),
                           dim3(256), 0, s, p);
    }
    hipLaunchKernelGGL((ssm::bwd_main_kernel<T, DISC, CPLX, LPC>), chunk_grid, dim3(256), 0, s, p);
}

template <typename T, int LPC>
void launch_bwd_modes(const ssm_scan_desc_t* d, const ssm::BwdParams& p, dim3 grid, dim3 cgrid, hipStream_t s) {
    if (d->is_complex) {
        if (d->disc == SSM_DISC_EXP_EULER)
            launch_bwd_kernels<T, ssm::kEuler, true, LPC>(p, grid, cgrid, s);
        else
            launch_bwd_kernels<T, ssm::kTrap, true, LPC>(p, grid, cgrid, s);
    } else {
        if (d->disc == SSM_DISC_ZOH)
            launch_bwd_kernels<T, ssm::kZOH, false, LPC>(p, grid, cgrid, s);
        else if (d->disc == SSM_DISC_EXP_EULER)
            launch_bwd_kernels<T, ssm::kEuler, false, LPC>(p, grid, cgrid, s);
        else
            launch_bwd_kernels<T, ssm::kTrap, false, LPC>(p, grid, cgrid, s);
    }
}

// lanes per channel of the backward kernels: 16 (N <= 16) or 64
int bwd_lpc(const ssm_scan_desc_t* d) { return d->dstate <= 16 ? 16 : 64; }

// waves per time chunk: 64 / lpc channels of one batch row per wave
int64_t bwd_waves(const ssm_scan_desc_t* d) {
    const int64_t cpw = 64 / bwd_lpc(d);
    return d->batch * ((d->dim + cpw - 1) / cpw);
}

template <typename T>
int launch_bwd(const ssm_scan_desc_t* d, const ssm::BwdParams& p, hipStream_t s) {
    const int64_t waves = bwd_waves(d);
    const int64_t blocks = (waves + 3) / 4, chunk_blocks = (waves * p.nchunks + 3) / 4;
    if (chunk_blocks > INT32_MAX || (d->batch * d->dim * d->dstate + 255) / 256 > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    const int64_t cw = d->is_complex ? 2 : 1;
    const int64_t na = d->dim * d->dstate, nb = d->batch * d->seqlen * d->dstate * cw, nd = p.dD ? d->dim : 0;
    int64_t zb = (na + 2 * nb + nd + 255) / 256;
    if (zb > 16384) zb = 16384;
    hipLaunchKernelGGL(ssm::bwd_zero_kernel, dim3(static_cast<unsigned>(zb)), dim3(256), 0, s, p.dA, na, p.dB, nb,
                       p.dC, nb, p.dD, nd);
    const dim3 grid(static_cast<unsigned>(blocks)), cgrid(static_cast<unsigned>(chunk_blocks));
    if (p.lpc == 16)
        launch_bwd_modes<T, 16>(d, p, grid, cgrid, s);
    else
        launch_bwd_modes<T, 64>(d, p, grid, cgrid, s);
    return hip_status(hipGetLastError());
}

// Time chunks of the reverse sweep: as many (of at least 256 steps, whole
// segments) as it takes to give the GPU about 2^19 lanes, eight waves per
// SIMD on 256 compute units; one chunk for a problem that wide on its own.
void bwd_chunking(const ssm_scan_desc_t* d, int64_t* chunk, int64_t* nchunks) {
    constexpr int64_t kTargetLanes = int64_t(1) << 19, kMinChunk = 256;
    const int64_t lanes = bwd_waves(d) * 64;
    int64_t want = (kTargetLanes + lanes - 1) / lanes;
    const int64_t most = (d->seqlen + kMinChunk - 1) / kMinChunk;
    if (want > most) want = most;
    if (want < 1) want = 1;
    int64_t c = (d->seqlen + want - 1) / want;
    c = (c + ssm::bwd::kSeg - 1) / ssm::bwd::kSeg * ssm::bwd::kSeg;
    *chunk = c;
    *nchunks = (d->seqlen + c - 1) / c;
}

// the snapshots, then the chunk adjoints (when there is more than one chunk)
size_t bwd_ckpt_bytes(const ssm_scan_desc_t* d) {
    const int64_t nseg = (d->seqlen + ssm::bwd::kSeg - 1) / ssm::bwd::kSeg;
    return static_cast<size_t>(ssm::round256(nseg * d->batch * d->dim * d->dstate * (d->is_complex ? 8 : 4)));
}

size_t bwd_workspace(const ssm_scan_desc_t* d) {
    int64_t chunk, n;
    bwd_chunking(d, &chunk, &n);
    const int64_t adj = n > 1 ? n * d->batch * d->dim * d->dstate * (d->is_complex ? 16 : 8) : 0;
    return bwd_ckpt_bytes(d) + static_cast<size_t>(adj);
}

int check_ssd_desc(const ssm_ssd_desc_t* d) {
    if (!d) return SSM_ERR_INVALID_ARGUMENT;
    if (d->batch < 1 || d->seqlen < 1 || d->dim < 1 || d->dstate < 1 || d->headdim < 1)
        return SSM_ERR_INVALID_ARGUMENT;
    if (d->io_dtype != SSM_DTYPE_F32 && d->io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
    if (d->io_dtype != SSM_DTYPE_BF16 || d->headdim != ssm::ssd::kP || d->dim % d->headdim != 0 ||
        d->dstate > ssm::ssd::kMaxN)
        return SSM_ERR_UNSUPPORTED;
    int64_t r;
    if (__builtin_mul_overflow(d->batch, d->seqlen, &r) || __builtin_mul_overflow(r, d->dim, &r) ||
        __builtin_mul_overflow(r, int64_t(8), &r))
        return SSM_ERR_INVALID_ARGUMENT;
    return SSM_OK;
}

size_t ssd_workspace(const ssm_ssd_desc_t* d) {
    const int64_t H = d->dim / d->headdim, nC = (d->seqlen + ssm::ssd::kQ - 1) / ssm::ssd::kQ;
    const int64_t planes = d->batch * H * nC;
    return static_cast<size_t>(2 * ssm::round256(planes * d->dstate * d->headdim * 2) + ssm::round256(planes * 4));
}

// Pointer checks shared by the scan and the step: required inputs present,
// lambda exactly for the trapezoid, theta only for a complex state, every
// pointer aligned to its element.
int check_inputs(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* theta, const void* lambda, const void* y) {
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARGUMENT;
    if (trap != (lambda != nullptr)) return SSM_ERR_INVALID_ARGUMENT;
    if (!desc->is_complex && theta) return SSM_ERR_INVALID_ARGUMENT;
    const size_t es = desc->io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    const void* io_ptrs[] = {u, delta, B, C, theta, lambda, y};
    for (const void* q : io_ptrs)
        if (q && !aligned(q, es)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(A, 4) || (D && !aligned(D, 4))) return SSM_ERR_INVALID_ARGUMENT;
    return SSM_OK;
}

int check_mimo_desc(const ssm_mimo_desc_t* d) {
    if (!d) return SSM_ERR_INVALID_ARGUMENT;
    if (d->batch < 1 || d->seqlen < 1 || d->dim < 1 || d->dstate < 1 || d->rank < 1 || d->chunk < 0 ||
        d->reserved != 0)
        return SSM_ERR_INVALID_ARGUMENT;
    if (d->io_dtype != SSM_DTYPE_F32 && d->io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
    if (d->disc < SSM_DISC_ZOH || d->disc > SSM_DISC_EXP_TRAPEZOIDAL) return SSM_ERR_UNSUPPORTED;
    if (d->is_complex != 0 && d->is_complex != 1) return SSM_ERR_UNSUPPORTED;
    if (d->is_complex && d->disc == SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d->dstate > 64) return SSM_ERR_UNSUPPORTED;
    if (d->rank != 1 && d->rank != 2 && d->rank != 4 && d->rank != 8) return SSM_ERR_UNSUPPORTED;
    // byte offsets of [B][L][D][max(2N, R)] and [B][L][N][R][2] fp32 words fit an int64
    const int64_t wide = 2 * d->dstate > d->rank ? 2 * d->dstate : d->rank;
    int64_t r;
    if (__builtin_mul_overflow(d->batch, d->seqlen, &r) || __builtin_mul_overflow(r, d->dim, &r) ||
        __builtin_mul_overflow(r, wide, &r) || __builtin_mul_overflow(r, int64_t(4), &r))
        return SSM_ERR_INVALID_ARGUMENT;
    if (__builtin_mul_overflow(d->batch, d->seqlen, &r) || __builtin_mul_overflow(r, d->dstate, &r) ||
        __builtin_mul_overflow(r, d->rank, &r) || __builtin_mul_overflow(r, int64_t(8), &r))
        return SSM_ERR_INVALID_ARGUMENT;
    return SSM_OK;
}

// lanes per channel of the MIMO kernels: one per pair of states, at least one per output
int mimo_lpc(const ssm_mimo_desc_t* d) {
    const int l = next_pow2((d->dstate + 1) / 2);
    return l < d->rank ? static_cast<int>(d->rank) : l;
}

// Time chunks of the MIMO scan.  Every chunk but the last costs a second
// sweep (its decay product and end state, about 60 % of the output sweep's
// work), but many short chunks keep every SIMD busy with several waves and
// balance the load: cutting the sequence until there are 2^21 lanes (32
// workgroups per CU of a 256-CU GPU) measured fastest, 4.6 ms against
// 6.4 ms for one chunk on a 4 x 2560 x 8192 x 16, R = 4 problem (flat from
// 128- to 512-step chunks).  The length is rounded down to a power of two
// (316 steps measured 4 % slower than 256), at least 128 steps.  The caller
// can fix the chunk length instead.
void mimo_chunking(const ssm_mimo_desc_t* d, int64_t* chunk, int64_t* nchunks) {
    int64_t c = d->chunk;
    if (c == 0) {
        constexpr int64_t kTargetLanes = int64_t(1) << 21;
        const int64_t lanes = d->batch * d->dim * mimo_lpc(d);
        const int64_t want = (kTargetLanes + lanes - 1) / lanes;
        const int64_t len = (d->seqlen + want - 1) / want;
        c = 128;
        while (2 * c <= len) c *= 2;
        if (want <= 1) c = d->seqlen;  // wide enough as one chunk
    }
    if (c > d->seqlen) c = d->seqlen;
    *chunk = c;
    *nchunks = (d->seqlen + c - 1) / c;
}

size_t mimo_workspace(const ssm_mimo_desc_t* d) {
    int64_t chunk, n;
    mimo_chunking(d, &chunk, &n);
    return static_cast<size_t>((n - 1) * d->batch * d->dim * d->dstate * (d->is_complex ? 16 : 8));
}

// Pointer checks of the MIMO scan and step: required inputs, lambda exactly
// for the trapezoid, theta only for a complex state, and the alignment of
// the runs the kernels read (u and y rows of R elements, B and C rows of R
// (complex) elements, each read with loads of up to 16 bytes).
int check_mimo_inputs(const ssm_mimo_desc_t* d, const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* theta, const void* lambda, const void* y) {
    const bool trap = d->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARGUMENT;
    if (trap != (lambda != nullptr)) return SSM_ERR_INVALID_ARGUMENT;
    if (!d->is_complex && theta) return SSM_ERR_INVALID_ARGUMENT;
    const size_t es = d->io_dtype == SSM_DTYPE_F32 ? 4 : 2, cw = d->is_complex ? 2 : 1;
    const size_t ua = d->rank * es < 16 ? d->rank * es : 16, ba = d->rank * cw * es < 16 ? d->rank * cw * es : 16;
    if (!aligned(u, ua) || !aligned(y, ua) || !aligned(B, ba) || !aligned(C, ba)) return SSM_ERR_INVALID_ARGUMENT;
    const void* io_ptrs[] = {delta, theta, lambda};
    for (const void* q : io_ptrs)
        if (q && !aligned(q, es)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(A, 4) || (D && !aligned(D, 4))) return SSM_ERR_INVALID_ARGUMENT;
    return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_scan_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

int ssm_scan_last_hip_error(void) { return g_last_hip_error; }

const char* ssm_scan_status_string(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SSM_ERR_UNSUPPORTED: return "unsupported configuration";
        case SSM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SSM_ERR_HIP: return "HIP runtime error";
        case SSM_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

int ssm_scan_algo(const ssm_scan_desc_t* desc) {
    if (check_desc(desc) != SSM_OK) return -1;
    return choose_algo(desc);
}

size_t ssm_scan_workspace_bytes(const ssm_scan_desc_t* desc) {
    if (check_desc(desc) != SSM_OK) return 0;
    if (choose_algo(desc) != SSM_ALGO_CHUNKED) return 0;
    if (desc->dstate > ssm::kChunkLanes) return 0;
    return ssm::chunked_workspace_bytes(desc->batch, desc->seqlen, desc->dim);
}

int ssm_scan_fwd(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A,
                 const void* B, const void* C, const float* D, const void* theta, const void* lambda,
                 void* y, float* h_last, void* workspace, size_t workspace_bytes, void* stream) {
    return ssm_scan_fwd_ex(desc, u, delta, A, B, C, D, theta, lambda, nullptr, nullptr, y, h_last, nullptr,
                           workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_ex(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A,
                    const void* B, const void* C, const float* D, const void* theta, const void* lambda,
                    const float* h0, const float* q0, void* y, float* h_last, float* q_last, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st = check_desc(desc);
    if (st != SSM_OK) return st;
    st = check_inputs(desc, u, delta, A, B, C, D, theta, lambda, y);
    if (st != SSM_OK) return st;
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!trap && (q0 || q_last)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t ss = desc->is_complex ? 8 : 4;  // one state element
    const void* st_ptrs[] = {h0, q0, h_last, q_last};
    for (const void* q : st_ptrs)
        if (q && !aligned(q, ss)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t es = desc->io_dtype == SSM_DTYPE_F32 ? 4 : 2;

    const int algo = choose_algo(desc);
    if (algo == SSM_ALGO_CHUNKED && desc->dstate > ssm::kChunkLanes) return SSM_ERR_UNSUPPORTED;
    if (algo == SSM_ALGO_SWEEP && sweep_unsupported(desc)) return SSM_ERR_UNSUPPORTED;
    const size_t need = algo == SSM_ALGO_CHUNKED
                            ? ssm::chunked_workspace_bytes(desc->batch, desc->seqlen, desc->dim)
                            : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return SSM_ERR_INVALID_ARGUMENT;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (algo == SSM_ALGO_CHUNKED) {
        ssm::ChunkParams p{};
        p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta;
        p.lambda = lambda; p.y = y; p.h_last = h_last;
        p.h0 = h0; p.q0 = q0; p.q_last = q_last;
        p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
        p.workspace = workspace;
        p.theta_pairs = (desc->dstate % 2 == 0) && aligned(theta, 2 * es);
        p.rows_dma = (desc->dim * static_cast<int64_t>(es)) % 16 == 0 && aligned(u, 16) && aligned(delta, 16) &&
                     (!lambda || aligned(lambda, 16));
        st = desc->io_dtype == SSM_DTYPE_F32
                 ? ssm::launch_chunked<float>(desc->disc, desc->is_complex != 0, p, s)
                 : ssm::launch_chunked<uint16_t>(desc->disc, desc->is_complex != 0, p, s);
        return st < 0 ? hip_status(static_cast<hipError_t>(-st)) : st;
    }

    if (algo == SSM_ALGO_SWEEP) {
        ssm::SweepParams p{};
        p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta;
        p.lambda = lambda; p.y = y; p.h_last = h_last;
        p.h0 = h0; p.q0 = q0; p.q_last = q_last;
        p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
        const bool pairs = desc->is_complex && aligned(B, 2 * es) && aligned(C, 2 * es);
        return desc->io_dtype == SSM_DTYPE_F32 ? launch_sweep<float>(desc, p, pairs, s)
                                               : launch_sweep<uint16_t>(desc, p, pairs, s);
    }

    ssm::SeqParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta;
    p.lambda = lambda; p.y = y; p.h_last = h_last;
    p.h0 = h0; p.q0 = q0; p.q_last = q_last;
    p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
    p.lpc = next_pow2(desc->dstate);
    return desc->io_dtype == SSM_DTYPE_F32 ? launch_sequential<float>(desc, p, s)
                                           : launch_sequential<uint16_t>(desc, p, s);
}

int ssm_scan_fwd_noalloc(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* theta, const void* lambda,
                         void* y, float* h_last, void* stream) {
    // every check that needs no device first, so that invalid calls and
    // over-limit problems return before any HIP call
    int st = check_desc(desc);
    if (st != SSM_OK) return st;
    st = check_inputs(desc, u, delta, A, B, C, D, theta, lambda, y);
    if (st != SSM_OK) return st;
    if (h_last && !aligned(h_last, desc->is_complex ? 8 : 4)) return SSM_ERR_INVALID_ARGUMENT;
    const int algo = choose_algo(desc);
    if (algo == SSM_ALGO_CHUNKED && desc->dstate > ssm::kChunkLanes) return SSM_ERR_UNSUPPORTED;
    if (algo == SSM_ALGO_SWEEP && sweep_unsupported(desc)) return SSM_ERR_UNSUPPORTED;
    const size_t need =
        algo == SSM_ALGO_CHUNKED ? ssm::chunked_workspace_bytes(desc->batch, desc->seqlen, desc->dim) : 0;
    if (need > SSM_SCAN_NOALLOC_SCRATCH_BYTES) return SSM_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (!ws) return SSM_ERR_HIP;
    }
    return ssm_scan_fwd_ex(desc, u, delta, A, B, C, D, theta, lambda, nullptr, nullptr, y, h_last, nullptr, ws,
                           need > 0 ? SSM_SCAN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int ssm_scan_step(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                  const void* C, const float* D, const void* theta, const void* lambda, const void* u_prev,
                  const void* B_prev, float* h, void* y, void* stream) {
    int st = check_desc(desc);
    if (st != SSM_OK) return st;
    if (desc->seqlen != 1) return SSM_ERR_INVALID_ARGUMENT;
    st = check_inputs(desc, u, delta, A, B, C, D, theta, lambda, y);
    if (st != SSM_OK) return st;
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!h || !aligned(h, desc->is_complex ? 8 : 4)) return SSM_ERR_INVALID_ARGUMENT;
    if ((u_prev != nullptr) != (B_prev != nullptr) || (!trap && u_prev)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t es = desc->io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    if ((u_prev && !aligned(u_prev, es)) || (B_prev && !aligned(B_prev, es))) return SSM_ERR_INVALID_ARGUMENT;

    ssm::StepParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta;
    p.lambda = lambda; p.u_prev = u_prev; p.B_prev = B_prev; p.h = h; p.y = y;
    p.batch = desc->batch; p.dim = desc->dim; p.dstate = desc->dstate;
    p.lpc = next_pow2((desc->dstate + 1) / 2);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return desc->io_dtype == SSM_DTYPE_F32 ? launch_step<float>(desc, p, s) : launch_step<uint16_t>(desc, p, s);
}

size_t ssm_scan_bwd_workspace_bytes(const ssm_scan_desc_t* desc) {
    if (check_desc(desc) != SSM_OK) return 0;
    return bwd_workspace(desc);
}

int ssm_scan_bwd(const ssm_scan_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* theta, const void* lambda, const float* h0,
                 const void* dy, const float* dh_last, float* du, float* ddelta, float* dA, float* dB, float* dC,
                 float* dD, float* dtheta, float* dlambda, float* dh0, void* workspace, size_t workspace_bytes,
                 void* stream) {
    int st = check_desc(desc);
    if (st != SSM_OK) return st;
    st = check_inputs(desc, u, delta, A, B, C, D, theta, lambda, dy);
    if (st != SSM_OK) return st;
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!du || !ddelta || !dA || !dB || !dC) return SSM_ERR_INVALID_ARGUMENT;
    if (trap != (dlambda != nullptr)) return SSM_ERR_INVALID_ARGUMENT;
    if (dtheta && !theta) return SSM_ERR_INVALID_ARGUMENT;
    const float* f32[] = {du, ddelta, dA, dB, dC, dD, dtheta, dlambda};
    for (const float* q : f32)
        if (q && !aligned(q, 4)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t ss = desc->is_complex ? 8 : 4;
    const void* st_ptrs[] = {h0, dh_last, dh0};
    for (const void* q : st_ptrs)
        if (q && !aligned(q, ss)) return SSM_ERR_INVALID_ARGUMENT;
    // per-step element strides inside a 32-step segment are 32-bit
    if (desc->dim * desc->dstate * ssm::bwd::kSeg >= (int64_t(1) << 31)) return SSM_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace(desc);
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 256)) return SSM_ERR_INVALID_ARGUMENT;

    ssm::BwdParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta; p.lambda = lambda;
    p.h0 = h0; p.dy = dy; p.dh_last = dh_last;
    p.du = du; p.ddelta = ddelta; p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.dtheta = dtheta;
    p.dlambda = dlambda; p.dh0 = dh0;
    p.ckpt = static_cast<float*>(workspace);
    p.adj = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_ckpt_bytes(desc));
    p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
    int64_t chunk, nchunks;
    bwd_chunking(desc, &chunk, &nchunks);
    if (nchunks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    p.chunk = chunk;
    p.nchunks = static_cast<int32_t>(nchunks);
    p.lpc = bwd_lpc(desc);
    p.wg_sum = p.lpc == 16 && ((desc->dim + 3) / 4) % 4 == 0;  // a batch row's waves (4 channels each) fill workgroups
    hipStream_t s = static_cast<hipStream_t>(stream);
    return desc->io_dtype == SSM_DTYPE_F32 ? launch_bwd<float>(desc, p, s) : launch_bwd<uint16_t>(desc, p, s);
}

size_t ssm_ssd_workspace_bytes(const ssm_ssd_desc_t* desc) {
    if (check_ssd_desc(desc) != SSM_OK) return 0;
    return ssd_workspace(desc);
}

int ssm_ssd_fwd(const ssm_ssd_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                const void* C, const float* D, void* y, float* h_last, void* workspace, size_t workspace_bytes,
                void* stream) {
    const int st = check_ssd_desc(desc);
    if (st != SSM_OK) return st;
    if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARGUMENT;
    const void* io_ptrs[] = {u, delta, B, C, y};
    for (const void* q : io_ptrs)
        if (!aligned(q, 2)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(u, 16) || !aligned(y, 16)) return SSM_ERR_INVALID_ARGUMENT;  // moved in 16-byte rows of 8 channels
    if (!aligned(A, 4) || (D && !aligned(D, 4)) || (h_last && !aligned(h_last, 4))) return SSM_ERR_INVALID_ARGUMENT;
    const size_t need = ssd_workspace(desc);
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 256)) return SSM_ERR_INVALID_ARGUMENT;

    ssm::SsdParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.y = y; p.h_last = h_last;
    p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
    p.heads = desc->dim / desc->headdim;
    p.bc_vec = desc->dstate % 8 == 0 && aligned(B, 16) && aligned(C, 16);
    p.nchunks = (desc->seqlen + ssm::ssd::kQ - 1) / ssm::ssd::kQ;
    const int64_t planes = p.batch * p.heads * p.nchunks;
    char* ws = static_cast<char*>(workspace);
    const uint64_t plane_bytes = ssm::round256(planes * p.dstate * ssm::ssd::kP * 2);
    p.S = reinterpret_cast<uint16_t*>(ws);
    p.Hin = reinterpret_cast<uint16_t*>(ws + plane_bytes);
    p.E = reinterpret_cast<float*>(ws + 2 * plane_bytes);
    if (planes > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    const int64_t pass_threads = p.batch * p.heads * p.dstate * ssm::ssd::kP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<unsigned>(planes));
    if (p.dstate <= 16)
        hipLaunchKernelGGL((ssm::ssd_state_kernel<uint16_t, 16>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((ssm::ssd_state_kernel<uint16_t, ssm::ssd::kMaxN>), grid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(ssm::ssd_pass_kernel, dim3(static_cast<unsigned>((pass_threads + 255) / 256)), dim3(256), 0, s,
                       p);
    if (p.dstate <= 16)
        hipLaunchKernelGGL((ssm::ssd_out_kernel<uint16_t, 16>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((ssm::ssd_out_kernel<uint16_t, ssm::ssd::kMaxN>), grid, dim3(256), 0, s, p);
    return hip_status(hipGetLastError());
}

size_t ssm_mimo_workspace_bytes(const ssm_mimo_desc_t* desc) {
    if (check_mimo_desc(desc) != SSM_OK) return 0;
    return mimo_workspace(desc);
}

int ssm_mimo_fwd(const ssm_mimo_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* theta, const void* lambda, const float* h0,
                 const float* q0, void* y, float* h_last, float* q_last, void* workspace, size_t workspace_bytes,
                 void* stream) {
    int st = check_mimo_desc(desc);
    if (st != SSM_OK) return st;
    st = check_mimo_inputs(desc, u, delta, A, B, C, D, theta, lambda, y);
    if (st != SSM_OK) return st;
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!trap && (q0 || q_last)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t ss = desc->is_complex ? 8 : 4;
    const void* st_ptrs[] = {h0, q0, h_last, q_last};
    for (const void* q : st_ptrs)
        if (q && !aligned(q, ss)) return SSM_ERR_INVALID_ARGUMENT;
    int64_t chunk, nchunks;
    mimo_chunking(desc, &chunk, &nchunks);
    const size_t need = mimo_workspace(desc);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 16)) return SSM_ERR_INVALID_ARGUMENT;
    }
    const int lpc = mimo_lpc(desc);
    const int64_t BD = desc->batch * desc->dim;
    const int64_t blocks = desc->batch * ((desc->dim * lpc + 255) / 256) * nchunks;
    if (nchunks > INT32_MAX || blocks > INT32_MAX || (BD * desc->dstate + 255) / 256 > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;

    ssm::MimoParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta; p.lambda = lambda;
    p.h0 = h0; p.q0 = q0; p.y = y; p.h_last = h_last; p.q_last = q_last;
    p.carry = static_cast<float*>(need > 0 ? workspace : nullptr);
    p.batch = desc->batch; p.seqlen = desc->seqlen; p.dim = desc->dim; p.dstate = desc->dstate;
    p.chunk = chunk; p.nchunks = static_cast<int32_t>(nchunks); p.lpc = lpc;
    return hip_status(ssm::launch_mimo_scan(p, desc->io_dtype == SSM_DTYPE_BF16, desc->disc, desc->is_complex != 0,
                                            static_cast<int>(desc->rank), static_cast<hipStream_t>(stream)));
}

int ssm_mimo_step(const ssm_mimo_desc_t* desc, const void* u, const void* delta, const float* A, const void* B,
                  const void* C, const float* D, const void* theta, const void* lambda, const void* u_prev,
                  const void* B_prev, float* h, void* y, void* stream) {
    int st = check_mimo_desc(desc);
    if (st != SSM_OK) return st;
    if (desc->seqlen != 1) return SSM_ERR_INVALID_ARGUMENT;
    st = check_mimo_inputs(desc, u, delta, A, B, C, D, theta, lambda, y);
    if (st != SSM_OK) return st;
    const bool trap = desc->disc == SSM_DISC_EXP_TRAPEZOIDAL;
    if (!h || !aligned(h, desc->is_complex ? 8 : 4)) return SSM_ERR_INVALID_ARGUMENT;
    if ((u_prev != nullptr) != (B_prev != nullptr) || (!trap && u_prev)) return SSM_ERR_INVALID_ARGUMENT;
    const size_t es = desc->io_dtype == SSM_DTYPE_F32 ? 4 : 2, cw = desc->is_complex ? 2 : 1;
    const size_t ua = desc->rank * es < 16 ? desc->rank * es : 16;
    const size_t ba = desc->rank * cw * es < 16 ? desc->rank * cw * es : 16;
    if ((u_prev && !aligned(u_prev, ua)) || (B_prev && !aligned(B_prev, ba))) return SSM_ERR_INVALID_ARGUMENT;
    const int lpc = mimo_lpc(desc);
    if (desc->batch * ((desc->dim * lpc + 255) / 256) > INT32_MAX) return SSM_ERR_UNSUPPORTED;

    ssm::MimoStepParams p{};
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = D; p.theta = theta; p.lambda = lambda;
    p.u_prev = u_prev; p.B_prev = B_prev; p.h = h; p.y = y;
    p.batch = desc->batch; p.dim = desc->dim; p.dstate = desc->dstate; p.lpc = lpc;
    p.pairs = desc->dstate % 2 == 0 && aligned(h, desc->is_complex ? 16 : 8);
    return hip_status(ssm::launch_mimo_step(p, desc->io_dtype == SSM_DTYPE_BF16, desc->disc, desc->is_complex != 0,
                                            static_cast<int>(desc->rank), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
