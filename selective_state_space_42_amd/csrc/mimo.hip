// mimo.hip -- the MIMO scan kernels' instantiations and launchers.  Kept in a
// translation unit of their own so the library's sources compile in parallel.
#include "kernel_mimo.h"

namespace ssm {
namespace {

template <typename T, int DISC, bool CPLX, int R>
hipError_t scan_r(const MimoParams& p, hipStream_t s) {
    const int64_t BD = p.batch * p.dim;
    const int64_t wgc = p.batch * ((p.dim * p.lpc + 255) / 256);  // workgroups per time chunk
    if (p.nchunks > 1) {
        hipLaunchKernelGGL((mimo_scan_kernel<T, DISC, CPLX, R, false>),
                           dim3(static_cast<unsigned>(wgc * (p.nchunks - 1))), dim3(256),
                           mimo_scan_lds_bytes(p.dstate, R, CPLX, false), s, p);
        const int64_t bdn = BD * p.dstate;
        hipLaunchKernelGGL((mimo_carry_kernel<CPLX>), dim3(static_cast<unsigned>((bdn + 255) / 256)), dim3(256), 0,
                           s, p);
    }
    hipLaunchKernelGGL((mimo_scan_kernel<T, DISC, CPLX, R, true>), dim3(static_cast<unsigned>(wgc * p.nchunks)),
                       dim3(256), mimo_scan_lds_bytes(p.dstate, R, CPLX, true), s, p);
    return hipGetLastError();
}

template <typename T, int DISC, bool CPLX, int R>
hipError_t step_r(const MimoStepParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.batch * ((p.dim * p.lpc + 255) / 256)));
    const size_t lds = mimo_step_lds_bytes(p.dstate, R, CPLX, DISC == kTrap);
    if (p.pairs)
        hipLaunchKernelGGL((mimo_step_kernel<T, DISC, CPLX, R, true>), grid, dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((mimo_step_kernel<T, DISC, CPLX, R, false>), grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

// rank and mode dispatch for either launcher
template <template <typename, int, bool, int> class Op, typename T, int DISC, bool CPLX, typename P>
hipError_t by_rank(const P& p, int rank, hipStream_t s) {
    switch (rank) {
        case 1: return Op<T, DISC, CPLX, 1>::run(p, s);
        case 2: return Op<T, DISC, CPLX, 2>::run(p, s);
        case 4: return Op<T, DISC, CPLX, 4>::run(p, s);
        case 8: return Op<T, DISC, CPLX, 8>::run(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <template <typename, int, bool, int> class Op, typename T, typename P>
hipError_t by_mode(const P& p, int disc, bool cplx, int rank, hipStream_t s) {
    if (cplx) {
        if (disc == kEuler) return by_rank<Op, T, kEuler, true>(p, rank, s);
        if (disc == kTrap) return by_rank<Op, T, kTrap, true>(p, rank, s);
        return hipErrorInvalidValue;
    }
    if (disc == kZOH) return by_rank<Op, T, kZOH, false>(p, rank, s);
    if (disc == kEuler) return by_rank<Op, T, kEuler, false>(p, rank, s);
    return by_rank<Op, T, kTrap, false>(p, rank, s);
}

template <typename T, int DISC, bool CPLX, int R>
struct ScanOp {
    static hipError_t run(const MimoParams& p, hipStream_t s) { return scan_r<T, DISC, CPLX, R>(p, s); }
};
template <typename T, int DISC, bool CPLX, int R>
struct StepOp {
    static hipError_t run(const MimoStepParams& p, hipStream_t s) { return step_r<T, DISC, CPLX, R>(p, s); }
};

}  // namespace

hipError_t launch_mimo_scan(const MimoParams& p, bool bf16, int disc, bool cplx, int rank, hipStream_t s) {
    return bf16 ? by_mode<ScanOp, uint16_t>(p, disc, cplx, rank, s) : by_mode<ScanOp, float>(p, disc, cplx, rank, s);
}

hipError_t launch_mimo_step(const MimoStepParams& p, bool bf16, int disc, bool cplx, int rank, hipStream_t s) {
    return bf16 ? by_mode<StepOp, uint16_t>(p, disc, cplx, rank, s) : by_mode<StepOp, float>(p, disc, cplx, rank, s);
}

}  // namespace ssm
