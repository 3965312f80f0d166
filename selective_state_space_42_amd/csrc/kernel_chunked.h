// kernel_chunked.h -- chunked scan with a decoupled look-back carry (in progress).
#pragma once

#include "device_common.h"

namespace ssm {

constexpr int kChunkLanes = 16;  // lanes per channel of the chunked kernel (max dstate)

struct ChunkParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;
    const void* theta;
    const void* lambda;
    void* y;
    float* h_last;
    int64_t batch, seqlen, dim, dstate;
    void* workspace;
};

inline bool chunked_preferred(int64_t, int64_t, int64_t) { return false; }
inline size_t chunked_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

template <typename T>
int launch_chunked(int, bool, const ChunkParams&, hipStream_t) { return SSM_ERR_UNSUPPORTED; }

}  // namespace ssm
