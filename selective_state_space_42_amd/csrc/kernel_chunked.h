// kernel_chunked.h -- the chunked scan: register-resident tiles along the
// sequence, combined by a decoupled look-back.
//
// Work decomposition
//   lane      = (channel c, state pair p): 8 lanes per channel, states
//               n = 2p, 2p+1 in each lane, 8 consecutive channels per wave.
//   wave      = 24 consecutive steps of those 8 channels.
//   tile (WG) = 4 waves = 96 consecutive steps x 8 channels.
// Tiles along the sequence are chained by the associative combine of the
// operator pairs (a, b) -> (a2 a1, a2 b1 + b2) (fengwang.github.io essay on
// the complex parallel scan, section on the mathematics of the parallel
// scan; the chunk-and-merge formulation is section 3 of the intelliparadigm
// article on selective scan).  Each tile is processed in two passes over
// registers:
//   pass 1  discretise every step (one exp and, for a complex state, one
//           sin/cos per element), keep alpha_t in VGPRs, run the recurrence
//           from a zero state to get the wave's aggregate (P = prod alpha,
//           h_loc); combine the 4 wave aggregates in LDS; publish the tile
//           aggregate; look back over predecessor tiles for the carry-in.
//   pass 2  rerun the recurrence from the true incoming state using the
//           stored alpha_t (no transcendental is evaluated twice) and form
//           y_t = Re(sum_n C_t[n] h_t[n]) + D u_t; the sum over n is reduced
//           through LDS, 8 steps at a time.
// The (B, L, D, N) state never reaches memory.
//
// Exponential-trapezoidal form.  With beta'_t = (1 - lambda_t) delta_t the
// recurrence h_t = alpha_t h_{t-1} + lambda_t delta_t q_t
// + beta'_t alpha_t q_{t-1} (q_t = B_t u_t) is carried in the shifted state
// g_t = h_t + beta'_{t+1} q_t, which obeys the exponential-Euler form
//   g_t = alpha_t g_{t-1} + w_t B_t,   w_t = (lambda_t delta_t + beta'_{t+1}) u_t,
// and y_t = Re(sum_n C_t g_t) + (D - beta'_{t+1} K_t) u_t with
// K_t = Re(sum_n C_t[n] B_t[n]); beta'_L = 0 so g_{L-1} = h_{L-1}.  This is the
// two-band (decay mask times two-band mask) structure the ai.tomabc.com
// Mamba-3 story describes for the exponential-trapezoidal discretisation.
//
// Cross-tile protocol (per channel group, tiles in sequence order):
//   flag 0 = nothing, 1 = aggregate (P, h_loc) published, 2 = inclusive state
//   published.  Tiles take tickets from one of 8 counters (one per XCD slot,
//   blockIdx % 8) so that a tile only ever waits on tiles that started earlier
//   (forward progress).  Flags move through relaxed agent-scope atomics and
//   payloads through loads and stores with the same coherent (sc1) cache
//   policy, which bypass the per-XCD L2 (coherent across XCDs); the
//   publisher waits for its payload stores to complete (s_waitcnt vmcnt(0))
//   before storing the flag, and readers load the payload only after seeing
//   the flag.  This avoids whole-L2 write-back/invalidate fences.
// A prep kernel zeroes flags and counters, converts B and C to fp32 rows of
// (B re, B im, C re, C im) per (b, t, n) (zero padded to whole tiles and to
// 16 states) and, for the trapezoid, computes K_t.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "device_math.h"

namespace ssm {

constexpr int kChunkLanes = 16;  // states covered by one channel's lanes (max dstate)

namespace chunk {
constexpr int kLPC = 8;            // lanes per channel
constexpr int kNPL = 2;            // states per lane
constexpr int kCPW = 64 / kLPC;    // channels per wave and per tile
constexpr int kWaves = 4;          // waves per workgroup, consecutive in time
constexpr int kTW = 24;            // steps per wave (a multiple of 8)
constexpr int kTT = kWaves * kTW;  // steps per tile
constexpr int kThreads = kWaves * 64;
constexpr int kCpolSc1 = 16;       // buffer-access cache policy: coherent across the device (as agent-scope atomics)
constexpr int kSlots = 8;          // ticket counters (one per XCD)
constexpr int kDmaWaves = kWaves - 1;  // waves 1.. issue the tile's LDS copies; wave 0 looks back
constexpr int kPayloadF2 = 3 * 64 * kNPL;  // float2 per tile: aggregate P, aggregate h, inclusive h
constexpr int kLookWindow = 16;            // predecessor flags read at once by the look-back
constexpr int kLookBatch = 1;              // predecessor payloads loaded at once
enum : uint32_t { kFlagEmpty = 0, kFlagAggregate = 1, kFlagInclusive = 2 };
}  // namespace chunk

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
    const float* h0;  // state before step 0, layout of h_last (NULL: zero)
    const float* q0;  // trapezoid: q_{-1} = B_{-1} u_{-1}, layout of h_last (NULL: zero)
    float* q_last;    // trapezoid: q_{L-1} = B_{L-1} u_{L-1} (written when not NULL)
    int64_t batch, seqlen, dim, dstate;
    void* workspace;
    int32_t theta_pairs;  // 1: dstate even and theta aligned to two elements
    int32_t rows_dma;     // 1: dim * element size a multiple of 16 and u, delta, lambda 16-byte aligned
                          //    (rows move by DMA in 16-byte chunks)
};

struct ChunkLayout {
    int64_t n_dblk;    // channel groups per batch row, ceil(D / kCPW)
    int64_t groups;    // batch * n_dblk
    int64_t n_tt;      // tiles along the sequence
    int64_t l_pad;     // n_tt * kTT
    int64_t slot_groups[chunk::kSlots];
    int64_t max_slot_tiles;
    uint64_t off_flags, off_payload, off_bc, off_k, total;
};

inline uint64_t round256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Channel groups of 8 are bundled by 8 (64 channels, one 128-byte row of the
// per-token arrays in bf16); bundle s goes to ticket slot s % 8.
inline ChunkLayout chunk_layout(int64_t B, int64_t L, int64_t D) {
    using namespace chunk;
    ChunkLayout l{};
    l.n_dblk = (D + kCPW - 1) / kCPW;
    l.groups = B * l.n_dblk;
    l.n_tt = (L + kTT - 1) / kTT;
    l.l_pad = l.n_tt * kTT;
    const int64_t full = l.groups / 8, rem = l.groups % 8;
    int64_t mx = 0;
    for (int s = 0; s < kSlots; ++s) {
        int64_t cnt = 8 * (full / kSlots + (s < full % kSlots ? 1 : 0));
        if (rem > 0 && s == full % kSlots) cnt += rem;
        l.slot_groups[s] = cnt;
        mx = cnt > mx ? cnt : mx;
    }
    l.max_slot_tiles = mx * l.n_tt;
    uint64_t off = 256;  // ticket counters
    l.off_flags = off;
    off += round256(uint64_t(l.groups * l.n_tt) * 4);
    l.off_payload = off;
    off += round256(uint64_t(l.groups * l.n_tt) * kPayloadF2 * 8);
    l.off_bc = off;
    off += round256(uint64_t(B * l.l_pad) * kChunkLanes * 16);
    l.off_k = off;
    off += round256(uint64_t(B * l.l_pad) * 4);
    l.total = off;
    return l;
}

inline size_t chunked_workspace_bytes(int64_t B, int64_t L, int64_t D) { return chunk_layout(B, L, D).total; }

// The chunked kernel fills the GPU whatever the channel count; the sequential
// kernel is kept for dstate > 16 and as an independent formulation.
inline bool chunked_preferred(int64_t, int64_t, int64_t) { return true; }

// ---------------------------------------------------------------- helpers

// vmcnt(0); the empty asm statements keep the compiler from moving memory
// operations across the wait
__device__ __forceinline__ void wait_stores() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

// Test builds only (SSM_LOOKBACK_TEST_DELAY > 0, see the build script): a
// bounded pause before a tile raises a flag, of 0 .. SSM_LOOKBACK_TEST_DELAY
// sleeps of 64 x 64 clocks chosen by a hash of the chain, the tile and the
// flag, so successors meet their predecessors' flags in scrambled orders
// (empty, aggregate or inclusive at any distance) while every wave still ends
// normally.  Compiles to nothing in the library.
#ifndef SSM_LOOKBACK_TEST_DELAY
#define SSM_LOOKBACK_TEST_DELAY 0
#endif
__device__ __forceinline__ void test_publish_delay(uint32_t chain, int64_t tile, uint32_t salt) {
    if constexpr (SSM_LOOKBACK_TEST_DELAY > 0) {
        uint32_t h = static_cast<uint32_t>(tile) * 2654435761u ^ (chain * 40503u + salt * 97u);
        h ^= h >> 15;
        h *= 0x2c1b3c6du;
        h ^= h >> 12;
        const int n = static_cast<int>(h % (SSM_LOOKBACK_TEST_DELAY + 1));
        for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(64);
    }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt(0)) but not for its global loads, stores or copies into LDS, which
// a __syncthreads() may wait for whenever any are in flight.  Used where
// those are deliberately left outstanding across the barrier; every reader of
// their results waits for them itself.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A buffer resource whose base and size the caller knows to be the same in
// every lane, declared so: read from the first lane into scalar registers.
// Without it a base picked from a small array by a (uniform) index stays in
// vector registers, and every access through the resource becomes a loop
// over the distinct values (v_readfirstlane, compare, masked access).
__device__ __forceinline__ rsrc_t make_uniform_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    const void* ub = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return make_rsrc(ub, __builtin_amdgcn_readfirstlane(bytes));
}

// byte offset of (section, lane, state j) in a tile's payload
__device__ __forceinline__ uint32_t pay_off(int section, int lane, int j) {
    return static_cast<uint32_t>(((section * 64 + lane) * chunk::kNPL + j) * 8);
}

// A lane's two states of one payload section move as one 16-byte access at a
// wave-uniform tile base, so that one instruction covers a whole 1 KB
// section (8-byte accesses per state left every line half written per
// instruction, and the coherent stores went out as partial lines, twice).
// The sc1 cache policy makes them coherent across the XCDs' L2s, as the
// flags' agent-scope atomics are.  No reader needs them to be atomic: a
// payload is read only after its flag, which is raised once the payload
// stores have completed.
typedef uint32_t pay_u32x4 __attribute__((ext_vector_type(4)));
static_assert(chunk::kNPL == 2, "two states of a lane are one 16-byte payload entry");
__device__ __forceinline__ void st_pay(float2* tile, int section, int lane, float2 s0, float2 s1) {
    const pay_u32x4 v = {__float_as_uint(s0.x), __float_as_uint(s0.y), __float_as_uint(s1.x), __float_as_uint(s1.y)};
    __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(tile, chunk::kPayloadF2 * 8), pay_off(section, lane, 0), 0,
                                           chunk::kCpolSc1);
}
__device__ __forceinline__ void ld_pay(const float2* tile, int section, int lane, float2* s0, float2* s1) {
    const pay_u32x4 v =
        __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(tile, chunk::kPayloadF2 * 8), pay_off(section, lane, 0), 0,
                                              chunk::kCpolSc1);
    *s0 = make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
    *s1 = make_float2(__uint_as_float(v.z), __uint_as_float(v.w));
}

struct Cx {
    float re, im;
};
__device__ __forceinline__ Cx cmul(Cx a, Cx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
__device__ __forceinline__ Cx cfma(Cx a, Cx b, Cx c) {  // a*b + c
    return {a.re * b.re - a.im * b.im + c.re, a.re * b.im + a.im * b.re + c.im};
}
__device__ __forceinline__ Cx to_cx(float2 v) { return {v.x, v.y}; }
__device__ __forceinline__ float2 to_f2(Cx v) { return make_float2(v.re, v.im); }

// ---------------------------------------------------------------- prep kernel

template <typename T, bool CPLX, bool TRAP>
__global__ void __launch_bounds__(256) chunk_prep_kernel(ChunkParams p, ChunkLayout lay) {
    using E = Elem<T>;
    char* ws = static_cast<char*>(p.workspace);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + lay.off_flags);
    float4* bc = reinterpret_cast<float4*>(ws + lay.off_bc);
    float* kt = reinterpret_cast<float*>(ws + lay.off_k);
    const T* Bm = static_cast<const T*>(p.B);
    const T* Cm = static_cast<const T*>(p.C);

    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    if (gtid < chunk::kSlots) ctrl[gtid] = 0;
    const int64_t nflags = lay.groups * lay.n_tt;
    for (int64_t i = gtid; i < nflags; i += stride) flags[i] = chunk::kFlagEmpty;

    // rows of kChunkLanes entries; stride is a multiple of 16 so each row's
    // 16 lanes stay together for the K_t reduction
    const int64_t items = p.batch * lay.l_pad * kChunkLanes;
    for (int64_t i = gtid; i < items; i += stride) {
        const int64_t row = i / kChunkLanes;
        const int n = static_cast<int>(i % kChunkLanes);
        const int64_t b = row / lay.l_pad, t = row % lay.l_pad;
        float br = 0.f, bi = 0.f, cr = 0.f, ci = 0.f;
        if (t < p.seqlen && n < p.dstate) {
            const int64_t k = (b * p.seqlen + t) * p.dstate + n;
            if constexpr (CPLX) {
                br = E::load(Bm, 2 * k);
                bi = E::load(Bm, 2 * k + 1);
                cr = E::load(Cm, 2 * k);
                ci = E::load(Cm, 2 * k + 1);
            } else {
                br = E::load(Bm, k);
                cr = E::load(Cm, k);
            }
        }
        // stored state-pair-major (entry j * kLPC + p for state n = p * kNPL + j)
        // so that a wave's reads of one entry per lane hit distinct LDS banks
        bc[row * kChunkLanes + (n % chunk::kNPL) * chunk::kLPC + n / chunk::kNPL] = make_float4(br, bi, cr, ci);
        if constexpr (TRAP) {
            float part = cr * br - ci * bi;  // Re(C B)
            for (int off = 8; off > 0; off >>= 1) part += __shfl_xor(part, off, 16);
            if (n == 0) kt[row] = part;
        }
    }

    // q_{L-1} = B_{L-1} u_{L-1} per (b, d, n): the trapezoid's input term that a
    // continuation of the sequence needs (bf16 products are exact in fp32)
    if constexpr (TRAP) {
        if (p.q_last) {
            const T* u = static_cast<const T*>(p.u);
            const int64_t nq = p.batch * p.dim * p.dstate;
            for (int64_t i = gtid; i < nq; i += stride) {
                const int64_t n = i % p.dstate, bd = i / p.dstate;
                const int64_t b = bd / p.dim, d = bd % p.dim;
                const int64_t t = p.seqlen - 1;
                const float x = E::load(u, (b * p.seqlen + t) * p.dim + d);
                const int64_t k = (b * p.seqlen + t) * p.dstate + n;
                if constexpr (CPLX) {
                    p.q_last[2 * i] = E::load(Bm, 2 * k) * x;
                    p.q_last[2 * i + 1] = E::load(Bm, 2 * k + 1) * x;
                } else {
                    p.q_last[i] = E::load(Bm, k) * x;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- main kernel

// Coordinates of one tile (uniform across the workgroup).  32-bit fields keep
// the scalar registers a persistent loop carries few.
struct Tile {
    uint32_t tt;  // tile index along the sequence
    uint32_t g;   // channel group
    uint32_t b;   // batch row
    uint32_t d0;  // first channel
    int nch;      // channels of the group that exist (<= kCPW)
    __device__ __forceinline__ int64_t t0() const { return int64_t(tt) * chunk::kTT; }  // first step
};

__device__ __forceinline__ Tile decode_tile(uint32_t local, uint32_t per_tt, int slot, const ChunkLayout& lay,
                                            int64_t D) {
    using namespace chunk;
    Tile t;
    const uint32_t tt = local / per_tt, r = local % per_tt;
    const uint32_t g = ((r / 8) * kSlots + slot) * 8 + (r % 8);
    const uint32_t ndb = static_cast<uint32_t>(lay.n_dblk);
    t.tt = tt;
    t.g = g;
    t.b = g / ndb;
    t.d0 = (g % ndb) * kCPW;
    t.nch = static_cast<int>(D - t.d0 < kCPW ? D - t.d0 : kCPW);
    return t;
}

// theta of one lane for one wave's steps, as loaded: bf16 keeps the (n, n+1)
// pair packed in one register; fp32 keeps two values.
template <typename T>
struct ThetaRegs;
template <>
struct ThetaRegs<uint16_t> {
    uint32_t w[chunk::kTW];
    __device__ __forceinline__ float get(int s, int j) const { return j ? bf16_hi(w[s]) : bf16_lo(w[s]); }
    __device__ __forceinline__ void pin(int s) { ssm::pin(w[s]); }
};
template <>
struct ThetaRegs<float> {
    float v[chunk::kTW][2];
    __device__ __forceinline__ float get(int s, int j) const { return v[s][j]; }
    __device__ __forceinline__ void pin(int s) {
        ssm::pin(v[s][0]);
        ssm::pin(v[s][1]);
    }
};

// ---- staging of one tile
//
// Registers carried from the issue of a tile's loads to their use.
template <typename T>
struct TileRegs {
    float a_ld[chunk::kNPL];  // A of this lane's states
    ThetaRegs<T> th;          // theta of this lane's states, this wave's steps
    float dskip;              // D of this thread's staging channel (tid % kCPW)
};

// Raw per-step rows in LDS, exactly as stored in memory: for each of the
// arrays u, delta, lambda, rows t0 .. t0 + kTT (one row past the tile, for
// the trapezoid's next-step terms) of the group's kCPW channels.  They arrive
// by buffer-to-LDS DMA in 16-byte chunks, 64 per wave instruction.
template <typename T>
struct RawRows {
    static constexpr int kRowDw = chunk::kCPW * int(sizeof(T)) / 4;   // dwords per row
    static constexpr int kChunks = (chunk::kTT + 1) * kRowDw / 4;     // 16-byte chunks per array
    static constexpr int kInstr = (kChunks + 63) / 64;                // DMA instructions per array
    static constexpr int kArrayDw = kChunks * 4;                      // array size in dwords
    static constexpr int kKChunks = chunk::kTT / 4;                   // K_t rows (fp32) in chunks
    static_assert(kRowDw % 4 == 0 && chunk::kTT % 4 == 0 && kKChunks <= 64, "chunked rows");
};

// Issue the loads a wave keeps in registers for tile `t`: A of its states,
// D of its staging channel and theta of its states over its steps (theta as
// stored, decoded in pass 1).  Buffer resources cover exactly the valid data,
// so lanes and steps outside read 0 and no load needs a branch or a mask.
template <typename T, bool CPLX>
__device__ __forceinline__ void issue_own(TileRegs<T>& r, const ChunkParams& p, const Tile& t, int tid, int c,
                                          int pr, int s0) {
    using namespace chunk;
    using BE = Buf<T>;
    constexpr uint32_t es = BE::kSize;
    constexpr bool kFast = std::is_same_v<T, uint16_t>;
    const T* theta = static_cast<const T*>(p.theta);
    const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
    const bool cok = c < t.nch;
    {
        const rsrc_t rA = make_rsrc(p.A + t.d0 * N, static_cast<uint32_t>(t.nch * N * 4));
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
            const int n = pr * kNPL + j;
            r.a_ld[j] = Buf<float>::load(rA, cok && n < N ? static_cast<uint32_t>((c * N + n) * 4) : kOutOfRange);
        }
        const rsrc_t rDs = make_rsrc(p.Dskip ? p.Dskip + t.d0 : p.A, p.Dskip ? static_cast<uint32_t>(t.nch * 4) : 0u);
        r.dskip = Buf<float>::load(rDs, static_cast<uint32_t>(tid % kCPW) * 4);
    }
    if constexpr (CPLX) {
        const int64_t ws0 = t.t0() + s0;  // this wave's first step
        const int64_t vsteps = L - ws0 < 0 ? 0 : (L - ws0 > kTW ? kTW : L - ws0);
        const uint32_t row = static_cast<uint32_t>(D * N) * es;
        const rsrc_t rT = make_rsrc(theta + ((t.b * L + (vsteps ? ws0 : 0)) * D + t.d0) * N,
                                    theta ? static_cast<uint32_t>(vsteps) * row : 0u);
        const int n0 = pr * kNPL;
        const uint32_t lo0 = cok && n0 < N ? static_cast<uint32_t>(c * N + n0) * es : kOutOfRange;
        const uint32_t lo1 = cok && n0 + 1 < N ? static_cast<uint32_t>(c * N + n0 + 1) * es : kOutOfRange;
        // one branch for the whole wave-tile, so the loads issue back to back
        if (p.theta_pairs) {  // N even: (n, n+1) adjacent and one element pair apart
#pragma unroll
            for (int s = 0; s < kTW; ++s) {
                if constexpr (kFast)
                    r.th.w[s] = __builtin_amdgcn_raw_buffer_load_b32(rT, lo0 + s * row, 0, 0);
                else
                    BE::load_pair(rT, lo0 + s * row, &r.th.v[s][0], &r.th.v[s][1]);
            }
        } else {
#pragma unroll
            for (int s = 0; s < kTW; ++s) {
                if constexpr (kFast) {
                    const uint32_t a = __builtin_amdgcn_raw_buffer_load_b16(rT, lo0 + s * row, 0, 0);
                    const uint32_t bb = __builtin_amdgcn_raw_buffer_load_b16(rT, lo1 + s * row, 0, 0);
                    r.th.w[s] = a | (bb << 16);
                } else {
                    r.th.v[s][0] = BE::load(rT, lo0 + s * row);
                    r.th.v[s][1] = BE::load(rT, lo1 + s * row);
                }
            }
        }
    }
}

// Pass-2 step after whose outputs a wave issues the next tile's register
// loads (after an output block: one per 8 steps).
constexpr int kOwnIssueStep = 7;
static_assert(kOwnIssueStep % 8 == 7 && kOwnIssueStep < chunk::kTW, "issue after an output block");

// Issue one DMA wave's share (dw in [0, kDmaWaves)) of tile `t`'s
// buffer-to-LDS copies: the B/C rows and, with p.rows_dma, the raw per-step
// rows and K_t.  With p.rows_dma == 0 (other D or unaligned pointers) the raw
// rows are instead loaded element by element in commit_tile().
template <typename T, int DISC>
__device__ __forceinline__ void issue_dma(const ChunkParams& p, const ChunkLayout& lay, const Tile& t, int lane,
                                          int dw, float4* s_bc_dst, uint32_t* s_raw, float* s_k) {
    using namespace chunk;
    using RR = RawRows<T>;
    constexpr uint32_t es = sizeof(T);
    constexpr bool kTR = DISC == kTrap;
    const float4* bc = reinterpret_cast<const float4*>(static_cast<const char*>(p.workspace) + lay.off_bc);
    const float* kt = reinterpret_cast<const float*>(static_cast<const char*>(p.workspace) + lay.off_k);
    const int64_t L = p.seqlen, D = p.dim;
    // B/C rows: each instruction fills 64 consecutive float4 entries
    {
        const float4* src = bc + (t.b * lay.l_pad + t.t0()) * kChunkLanes;
        constexpr int kInstr = kTT * kChunkLanes / 64;
#pragma unroll
        for (int k = 0; k < (kInstr + kDmaWaves - 1) / kDmaWaves; ++k) {
            const int q = k * kDmaWaves + dw;  // this wave's instruction (uniform)
            if (kInstr % kDmaWaves == 0 || q < kInstr)
                __builtin_amdgcn_global_load_lds(src + q * 64 + lane,
                                                 (__attribute__((address_space(3))) void*)(s_bc_dst + q * 64), 16, 0, 0);
        }
    }
    if (p.rows_dma) {
        // rows t0 .. t0 + rows - 1 exist (rows >= 1).  D * sizeof(T) and the
        // pointers are multiples of 16 bytes, so every 16-byte chunk of a row
        // lies wholly inside or wholly outside the resource's window.
        const int64_t rows = L - t.t0() > kTT + 1 ? kTT + 1 : L - t.t0();
        const uint32_t bytes = static_cast<uint32_t>((rows - 1) * D + t.nch) * es;
        const int64_t base = (t.b * L + t.t0()) * D + t.d0;
        const T* arrs[3] = {static_cast<const T*>(p.u), static_cast<const T*>(p.delta),
                            static_cast<const T*>(p.lambda)};
        constexpr int kArrays = kTR ? 3 : 2;
        constexpr int kTotal = kArrays * RR::kInstr + (kTR ? 1 : 0);
        constexpr int kRowChunks = RR::kRowDw / 4;
#pragma unroll
        for (int q = 0; q < (kTotal + kDmaWaves - 1) / kDmaWaves; ++q) {
            const int g = q * kDmaWaves + dw;  // this wave's DMA instruction (uniform)
            if (g < kArrays * RR::kInstr) {
                const int ar = g / RR::kInstr, iq = g % RR::kInstr;
                const int f = iq * 64 + lane;  // chunk of the array
                const int rw = f / kRowChunks, part = f % kRowChunks;
                const rsrc_t rs = make_uniform_rsrc(arrs[ar] + base, bytes);
                if (f < RR::kChunks)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rs, (__attribute__((address_space(3))) void*)(s_raw + ar * RR::kArrayDw + iq * 256), 16,
                        static_cast<uint32_t>(rw * D) * es + part * 16, 0, 0, 0);
            } else if (g < kTotal) {
                const rsrc_t rK = make_rsrc(kt + t.b * lay.l_pad + t.t0(), kTT * 4);
                if (lane < RR::kKChunks)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (__attribute__((address_space(3))) void*)(s_k), 16,
                                                             static_cast<uint32_t>(lane) * 16, 0, 0, 0);
            }
        }
    }
}

// Write the staged per-step terms of the current tile: (delta, w) and e per
// step and channel, from the raw rows in LDS (after they have landed and a
// workgroup barrier).  Without DMA the raw rows are first loaded element by
// element here (synchronously; followed by a barrier inside).
template <typename T, int DISC>
__device__ __forceinline__ void commit_tile(const TileRegs<T>& r, const ChunkParams& p, const ChunkLayout& lay,
                                            const Tile& t, int tid, uint32_t* s_raw, float* s_k,
                                            float2 (*s_dw)[chunk::kCPW], float (*s_e)[chunk::kCPW]) {
    using namespace chunk;
    using BE = Buf<T>;
    using RR = RawRows<T>;
    constexpr uint32_t es = BE::kSize;
    constexpr bool kTR = DISC == kTrap;
    const int64_t L = p.seqlen, D = p.dim;
    // [array][row][kCPW] stored bit patterns, arrays RR::kArrayDw dwords apart
    using RawT = std::conditional_t<sizeof(T) == 2, uint16_t, uint32_t>;
    RawT* raw = reinterpret_cast<RawT*>(s_raw);
    constexpr int kArrayEl = RR::kArrayDw * 4 / int(sizeof(T));
    const int cc = tid % kCPW;
    if (!p.rows_dma) {
        const int64_t rows = L - t.t0() > kTT + 1 ? kTT + 1 : L - t.t0();
        const uint32_t bytes = static_cast<uint32_t>((rows - 1) * D + t.nch) * es;
        const int64_t base = (t.b * L + t.t0()) * D + t.d0;
        const T* arrs[3] = {static_cast<const T*>(p.u), static_cast<const T*>(p.delta),
                            static_cast<const T*>(p.lambda)};
        constexpr int kArrays = kTR ? 3 : 2;
        const float* kt = reinterpret_cast<const float*>(static_cast<const char*>(p.workspace) + lay.off_k);
        for (int i = tid; i < (kTT + 1) * kCPW; i += kThreads) {
            const int rw = i / kCPW, ch = i % kCPW;
            const uint32_t off = ch < t.nch ? static_cast<uint32_t>(rw * D + ch) * es : kOutOfRange;
#pragma unroll
            for (int ar = 0; ar < kArrays; ++ar)
                raw[ar * kArrayEl + i] = static_cast<RawT>(BE::load_raw(make_rsrc(arrs[ar] + base, bytes), off));
        }
        if constexpr (kTR)
            for (int i = tid; i < kTT; i += kThreads) s_k[i] = kt[t.b * lay.l_pad + t.t0() + i];
        __syncthreads();
    }
    float dsk = r.dskip;
    pin(dsk);
#pragma unroll
    for (int k = 0; k < kTT * kCPW / kThreads; ++k) {
        // No validity test: rows past the sequence end arrive as zeros (and
        // K_t is zero there), so their terms come out zero; entries of
        // channels past the group's end are never read by a lane that stores.
        const int i = tid + k * kThreads;
        const int st = i / kCPW;
        const float x = BE::widen(raw[0 * kArrayEl + i]);
        const float dt = BE::widen(raw[1 * kArrayEl + i]);
        float w, e;
        if constexpr (DISC == kZOH) {
            w = x;
            e = dsk * x;
        } else if constexpr (DISC == kEuler) {
            w = dt * x;
            e = dsk * x;
        } else {
            const float lam = BE::widen(raw[2 * kArrayEl + i]);
            const float dn = BE::widen(raw[1 * kArrayEl + i + kCPW]);
            const float ln = BE::widen(raw[2 * kArrayEl + i + kCPW]);
            const float bnext = (1.f - ln) * dn;  // beta'_{t+1} (zero past the end)
            w = (lam * dt + bnext) * x;
            e = (dsk - bnext * s_k[st]) * x;
        }
        s_dw[st][cc] = make_float2(dt, w);
        s_e[st][cc] = e;
    }
}

// Wait until at most N vector-memory instructions of this wave are
// outstanding.  vmcnt retires in issue order, so this waits for everything
// issued before the last N.  The empty asm statements keep the compiler from
// moving memory operations across the wait.
template <int N>
__device__ __forceinline__ void wait_vm_below() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
    asm volatile("" ::: "memory");
}

// Tile aggregate (P, h) of one lane's states from the waves' aggregates in
// LDS, folded in step order: (P, h) <- (P_w P, P_w h + h_w).
__device__ __forceinline__ void tile_aggregate(const float2* s_aggP, const float2* s_aggH, int lane, Cx* Pt,
                                               Cx* Ht) {
    using namespace chunk;
#pragma unroll
    for (int j = 0; j < kNPL; ++j) {
        Pt[j] = {1.f, 0.f};
        Ht[j] = {0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const Cx Pw = to_cx(s_aggP[(w * 64 + lane) * kNPL + j]);
            Ht[j] = cfma(Pw, Ht[j], to_cx(s_aggH[(w * 64 + lane) * kNPL + j]));
            Pt[j] = cmul(Pw, Pt[j]);
        }
    }
}

// Carry-in (state after the last step before tile tt) of one chain, by one
// wave: read the flags of up to kLookWindow predecessors at once (one lane
// each), fold the aggregates of those that precede the nearest inclusive
// state (nearest first), then that inclusive state.  An empty flag before the
// nearest inclusive state stops the fold there; the rest is retried after a
// short sleep.  Tile 0 of a chain always publishes an inclusive state and
// every predecessor belongs to a running workgroup (see the kernel), so the
// loop ends.
__device__ __forceinline__ void look_back(const uint32_t* flag, const float2* pay_base, int64_t tt, int lane,
                                          Cx* carry) {
    using namespace chunk;
    Cx Pacc[kNPL], Hacc[kNPL];
#pragma unroll
    for (int j = 0; j < kNPL; ++j) {
        Pacc[j] = {1.f, 0.f};
        Hacc[j] = {0.f, 0.f};
    }
    int64_t k0 = tt - 1;  // nearest predecessor not folded yet
    for (;;) {
        const int64_t k = k0 - lane;
        const bool valid = lane < kLookWindow && k >= 0;
        uint32_t f = kFlagEmpty;
        if (valid) f = __hip_atomic_load(&flag[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t inc = __ballot(valid && f == kFlagInclusive);
        const uint64_t emp = __ballot(valid && f == kFlagEmpty);
        const int ni = inc ? __builtin_ctzll(inc) : 64;  // nearest inclusive
        const int ne = emp ? __builtin_ctzll(emp) : 64;  // nearest empty
        const bool found = ni < ne;                      // ni < kLookWindow then
        const int nagg = found ? ni : (ne < kLookWindow ? ne : kLookWindow);
        // fold nagg aggregates (and the inclusive state if found), loading
        // kLookBatch predecessors' payloads at a time
        int h0 = 0;
        do {
            const int nb = nagg - h0 < kLookBatch ? nagg - h0 : kLookBatch;
            const bool last = h0 + nb == nagg;
            float2 Pv[kLookBatch][kNPL], Hv[kLookBatch][kNPL], Iv[kNPL];
#pragma unroll
            for (int q = 0; q < kLookBatch; ++q) {
                if (q < nb) {
                    const float2* pk = pay_base + (k0 - h0 - q) * kPayloadF2;
                    ld_pay(pk, 0, lane, &Pv[q][0], &Pv[q][1]);
                    ld_pay(pk, 1, lane, &Hv[q][0], &Hv[q][1]);
                }
            }
            if (last && found) {
                const float2* pk = pay_base + (k0 - ni) * kPayloadF2;
                ld_pay(pk, 2, lane, &Iv[0], &Iv[1]);
            }
#pragma unroll
            for (int q = 0; q < kLookBatch; ++q) {
                if (q < nb) {
#pragma unroll
                    for (int j = 0; j < kNPL; ++j) {
                        Hacc[j] = cfma(Pacc[j], to_cx(Hv[q][j]), Hacc[j]);
                        Pacc[j] = cmul(Pacc[j], to_cx(Pv[q][j]));
                    }
                }
            }
            if (last && found) {
#pragma unroll
                for (int j = 0; j < kNPL; ++j) carry[j] = cfma(Pacc[j], to_cx(Iv[j]), Hacc[j]);
                return;
            }
            h0 += nb;
        } while (h0 < nagg);
        k0 -= nagg;
        if (ne < kLookWindow && ne == nagg) __builtin_amdgcn_s_sleep(2);  // waiting on a predecessor
    }
}

// Pass 1 over one wave's steps: discretise every step, keep alpha_t in
// registers (al_i holds b_t on the real path), run the recurrence from a zero
// state (g) and sum delta and theta for the wave's decay product.  SC selects
// the sin/cos evaluation.  The sums are kept where they stay exact enough:
// with hardware sin/cos theta is summed as its reduced revolutions (bounded
// by the step count), otherwise delta and theta are summed in fp64.
template <typename T, int DISC, bool CPLX, int SC, typename Acc>
__device__ __forceinline__ void pass1(const TileRegs<T>& r, const float2 (*s_dw)[chunk::kCPW],
                                      const float4 (*s_bc)[kChunkLanes], int s0, int c, int pr, const float* a_prep,
                                      const float* a_raw, const float* inv_a, float (&al_r)[chunk::kTW][chunk::kNPL],
                                      float (&al_i)[chunk::kTW][chunk::kNPL], Cx* gl, Acc* sth, Acc& sdt) {
    using namespace chunk;
    // the next step's LDS operands are read one step ahead
    float2 nx_dw = s_dw[s0][c];
    float2 nx_b[kNPL];
#pragma unroll
    for (int j = 0; j < kNPL; ++j) {
        const float4 q = s_bc[s0][j * kLPC + pr];
        nx_b[j] = make_float2(q.x, q.y);
    }
#pragma unroll
    for (int s = 0; s < kTW; ++s) {
        const float2 tc4 = nx_dw;  // (delta, w)
        float2 cb[kNPL];
#pragma unroll
        for (int j = 0; j < kNPL; ++j) cb[j] = nx_b[j];
        if (s + 1 < kTW) {
            nx_dw = s_dw[s0 + s + 1][c];
#pragma unroll
            for (int j = 0; j < kNPL; ++j) {
                const float4 q = s_bc[s0 + s + 1][j * kLPC + pr];
                nx_b[j] = make_float2(q.x, q.y);
            }
        }
        sdt += static_cast<Acc>(tc4.x);
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
            const float4 bcq = make_float4(cb[j].x, cb[j].y, 0.f, 0.f);
            if constexpr (CPLX) {
                const float rho = exp_dA(tc4.x, a_prep[j]);
                const float thv = r.th.get(s, j);
                float sn, cs;
                if constexpr (SC == kSinCosHw) {
                    const float rev = __builtin_amdgcn_fractf(thv * kInv2Pi);
                    sin_cos_rev(rev, &sn, &cs);
                    sth[j] += rev;
                } else {
                    sin_cos<SC>(thv, &sn, &cs);
                    sth[j] += static_cast<Acc>(thv);
                }
                const Cx al = {rho * cs, rho * sn};
                al_r[s][j] = al.re;
                al_i[s][j] = al.im;
                gl[j] = cfma(al, gl[j], Cx{tc4.y * bcq.x, tc4.y * bcq.y});
            } else {
                float rho, bt;
                if constexpr (DISC == kZOH) {  // weight (e^{delta A} - 1)/A (delta at A = 0)
                    float em1;
                    exp_expm1(tc4.x * a_raw[j], tc4.x * a_prep[j], &rho, &em1);
                    bt = (a_raw[j] != 0.f ? em1 * inv_a[j] : tc4.x) * tc4.y * bcq.x;
                } else {
                    rho = exp_dA(tc4.x, a_prep[j]);
                    bt = tc4.y * bcq.x;
                }
                al_r[s][j] = rho;
                al_i[s][j] = bt;
                gl[j].re = rho * gl[j].re + bt;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Persistent workgroups: each takes tickets from its slot's counter until the
// slot's tiles are exhausted.  The pipeline per workgroup is
//   [tile k: commit staged values to LDS | pass 1]
//   [look-back of k | copies of tile k+1's rows into LDS]
//   [pass 2 of k, with tile k+1's register loads issued after its first outputs]
// so tile k+1's memory latency overlaps tile k's look-back and pass 2.  A
// tile only waits on tiles with smaller tickets of the same slot; each such
// tile is held by a running workgroup that is processing it or will process it
// right after its current (even smaller) ticket, so the smallest unfinished
// ticket always makes progress.
template <typename T, int DISC, bool CPLX>
__global__ void __launch_bounds__(chunk::kThreads, 2) chunk_scan_kernel(ChunkParams p_in, ChunkLayout lay_in) {
    using namespace chunk;
    // Parameters are read from the kernel-argument segment, through a pointer
    // the compiler must treat as changed at the top of every tile.  Otherwise
    // it keeps every loop-invariant pointer and size in scalar registers for
    // the whole persistent loop, and the excess is spilled to vector lanes and
    // read back (v_readlane) in every tile's control code.  The arguments are
    // laid out in order at their natural alignment.
    using KArgs = const __attribute__((address_space(4))) char*;
    KArgs kargs = (KArgs)(__builtin_amdgcn_kernarg_segment_ptr());
    constexpr size_t kLayOff = (sizeof(ChunkParams) + alignof(ChunkLayout) - 1) / alignof(ChunkLayout) *
                               alignof(ChunkLayout);
    static_assert(std::is_trivially_copyable_v<ChunkParams> && std::is_standard_layout_v<ChunkParams> &&
                      std::is_trivially_copyable_v<ChunkLayout> && std::is_standard_layout_v<ChunkLayout>,
                  "the argument segment holds bitwise copies of the parameter structs");
    const ChunkParams& p = p_in;
    const ChunkLayout& lay = lay_in;
    using BE = Buf<T>;
    constexpr uint32_t es = BE::kSize;
    constexpr bool kFast = std::is_same_v<T, uint16_t>;
    constexpr bool kZ = DISC == kZOH;
    constexpr bool kTR = DISC == kTrap;
    static_assert(kTT * kChunkLanes % kThreads == 0 && kTT * kCPW % kThreads == 0, "tile shape");

    __shared__ float4 s_bcb[2][kTT][kChunkLanes];  // (B re, B im, C re, C im), double-buffered by tile
    __shared__ float2 s_dw[kTT][kCPW];         // (delta, w) per step and channel
    __shared__ float s_e[kTT][kCPW];           // e per step and channel (output's u term)
    __shared__ uint32_t s_raw[3 * RawRows<T>::kArrayDw];  // raw u, delta, lambda rows
    __shared__ float s_k[kTT];                              // K_t rows
    // pass-1 wave aggregates (P, h); once the incoming states are formed the
    // same space holds pass 2's y partials (kWaves x 8 steps x 64 lanes)
    // y partials: rows of 64 lanes padded to kRedRow floats, so that the
    // transposed reads (8 lanes of one channel, each from another row) fall
    // in distinct banks
    constexpr int kRedRow = 64 + 4;
    constexpr int kAggF2 = kWaves * 64 * kNPL;
    static_assert(2 * kAggF2 * 2 <= kWaves * 8 * kRedRow, "aggregate and partial buffers share space");
    __shared__ alignas(16) float s_x[kWaves * 8 * kRedRow];
    float2* s_aggP = reinterpret_cast<float2*>(s_x);           // [wave][lane][j]
    float2* s_aggH = reinterpret_cast<float2*>(s_x) + kAggF2;  // [wave][lane][j]
    float* s_red = s_x;                                         // [wave][step % 8][lane (padded)]
    __shared__ float2 s_carry[kWaves][64][kNPL];  // incoming state of each wave's steps
    __shared__ uint32_t s_ticket[2];  // the ticket after the current tile, by tile parity (buf)
    __shared__ uint32_t s_pred_inc;  // wave 0 holds the predecessor's inclusive state (see pred_flag)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int lane = tid & 63;
    const int c = lane / kLPC;
    const int pr = lane % kLPC;
    const int s0 = wave * kTW;  // this wave's first step within a tile
    const int slot = blockIdx.x % kSlots;
    const uint32_t per_tt = static_cast<uint32_t>(lay.slot_groups[slot]);
    const uint32_t slot_tiles = per_tt * static_cast<uint32_t>(lay.n_tt);

    TileRegs<T> r;  // one tile's register-carried loads

    // ---- prologue: first ticket, its loads, the ticket after it.  Later
    // tickets are requested in the carry step of the tile before the one that
    // reads them.
    uint32_t ticket = 0;  // thread 0: the ticket after the current tile (see the loop)
    if (tid == 0) {
        uint32_t* ctrl = static_cast<uint32_t*>(p.workspace);
        s_ticket[1] = __hip_atomic_fetch_add(&ctrl[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __hip_atomic_fetch_add(&ctrl[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    uint32_t cur = __builtin_amdgcn_readfirstlane(s_ticket[1]);
    if (cur >= slot_tiles) return;
    Tile tc = decode_tile(cur, per_tt, slot, lay, p.dim);
    int buf = 0;
    issue_own<T, CPLX>(r, p, tc, tid, c, pr, s0);
    if (wave != 0) issue_dma<T, DISC>(p, lay, tc, lane, wave - 1, &s_bcb[0][0][0], s_raw, s_k);
    // Wave 0: the flag of the current tile's predecessor as read in the carry
    // step of the previous tile (empty before the first tile).  A flag only rises, so
    // when it already showed the inclusive state the payload is loaded at the
    // start of the tile and has arrived by the time the look-back needs it.
    uint32_t pred_flag = kFlagEmpty;

    for (;;) {
        asm volatile("" : "+s"(kargs));
        const ChunkParams& p = *reinterpret_cast<const ChunkParams*>((const char*)kargs);
        const ChunkLayout& lay = *reinterpret_cast<const ChunkLayout*>((const char*)(kargs + kLayOff));
        const T* delta = static_cast<const T*>(p.delta);
        const T* lambda = static_cast<const T*>(p.lambda);
        T* y = static_cast<T*>(p.y);
        char* ws = static_cast<char*>(p.workspace);
        uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws);
        uint32_t* flags = reinterpret_cast<uint32_t*>(ws + lay.off_flags);
        float2* payload = reinterpret_cast<float2*>(ws + lay.off_payload);
        const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
        // ---- 1. stage the current tile
        wait_stores();  // this wave's loads and DMA (B/C rows, raw rows) have landed (vmcnt(0))
        __syncthreads();
        const bool pred_inc = tc.tt > 0 && __builtin_amdgcn_readfirstlane(pred_flag) == kFlagInclusive;  // wave 0 only
        float2 pred_state[kNPL];
        if (wave == 0 && pred_inc) {
            const float2* pk = payload + (tc.g * lay.n_tt + tc.tt - 1) * kPayloadF2;
            asm volatile("" ::: "memory");  // not above the flag test
            ld_pay(pk, 2, lane, &pred_state[0], &pred_state[1]);
        }
        if (tid == 0) {
            s_pred_inc = pred_inc ? 1u : 0u;
            s_ticket[buf] = ticket;  // read in this tile's carry step
        }
        commit_tile<T, DISC>(r, p, lay, tc, tid, s_raw, s_k, s_dw, s_e);
        __syncthreads();
        float4 (*s_bc)[kChunkLanes] = s_bcb[buf];

        // ---- 2. pass 1: discretise, keep alpha in registers, local aggregate
        const bool cok = c < tc.nch;
        const int64_t d = tc.d0 + (cok ? c : 0);
        bool nok[kNPL];
        float a_prep[kNPL], a_raw[kNPL], inv_a[kNPL];
#pragma unroll
        for (int s = 0; s < kTW; ++s) r.th.pin(s);
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
            nok[j] = cok && pr * kNPL + j < N;
            pin(r.a_ld[j]);
            a_raw[j] = r.a_ld[j];
            a_prep[j] = prep_A(a_raw[j]);
            inv_a[j] = a_raw[j] != 0.f ? 1.f / a_raw[j] : 0.f;
        }
        float al_r[kTW][kNPL], al_i[kTW][kNPL];  // alpha_t (al_i holds b_t on the real path)
        Cx gl[kNPL];
        using Acc = std::conditional_t<kFast, float, double>;  // sums of delta and theta
        Acc sth[kNPL], sdt = 0;
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
            gl[j] = {0.f, 0.f};
            sth[j] = 0;
        }
        if constexpr (kFast || !CPLX) {
            pass1<T, DISC, CPLX, kFast ? kSinCosHw : kSinCosPoly>(r, s_dw, s_bc, s0, c, pr, a_prep, a_raw, inv_a, al_r,
                                                                  al_i, gl, sth, sdt);
        } else {
            // fp32 complex state: the polynomial sin/cos when every |theta| of
            // this wave's steps is at most pi/4 (one uniform test per tile)
            float m = 0.f;
#pragma unroll
            for (int s = 0; s < kTW; ++s)
#pragma unroll
                for (int j = 0; j < kNPL; ++j) m = fmaxf(m, fabsf(r.th.get(s, j)));
            if (__any(!(m <= kPiOver4)))
                pass1<T, DISC, CPLX, kSinCosWide>(r, s_dw, s_bc, s0, c, pr, a_prep, a_raw, inv_a, al_r, al_i, gl, sth,
                                                 sdt);
            else
                pass1<T, DISC, CPLX, kSinCosPoly>(r, s_dw, s_bc, s0, c, pr, a_prep, a_raw, inv_a, al_r, al_i, gl, sth,
                                                  sdt);
        }
        // the wave's aggregate (P, h): P = prod alpha = exp(A sum delta) e^{i sum theta}
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
            const float mod = kFast ? exp_dA(static_cast<float>(sdt), a_prep[j])
                                    : static_cast<float>(exp(sdt * static_cast<double>(a_raw[j])));
            Cx P = {mod, 0.f};
            if constexpr (CPLX) {
                float sn, cs;
                if constexpr (kFast)
                    sin_cos_rev(__builtin_amdgcn_fractf(static_cast<float>(sth[j])), &sn, &cs);
                else
                    sin_cos_wide(static_cast<double>(sth[j]), &sn, &cs);
                P = {mod * cs, mod * sn};
            }
            s_aggP[(wave * 64 + lane) * kNPL + j] = to_f2(P);
            s_aggH[(wave * 64 + lane) * kNPL + j] = to_f2(gl[j]);
        }
        __syncthreads();

        // ---- 3. cross-tile carry.  Wave 0: look back, form the inclusive
        // state and every wave's incoming state.  Wave 1: publish the tile
        // aggregate.  Waves 1..: the next tile's LDS copies.  Then the ticket
        // after next and the next tile's predecessor flag.
        const uint32_t nx = __builtin_amdgcn_readfirstlane(s_ticket[buf]);
        const bool has_next = nx < slot_tiles;
        const Tile tn = has_next ? decode_tile(nx, per_tt, slot, lay, D) : tc;
        float2* pay_base = payload + (tc.g * lay.n_tt) * kPayloadF2;
        uint32_t* flag = flags + tc.g * lay.n_tt;
        const int64_t tt = tc.tt;
        float2* mine = pay_base + tt * kPayloadF2;
        if (wave != 0) {
            // The aggregate lets a successor that finds this tile before its
            // inclusive state fold past it.  When wave 0 already holds the
            // predecessor's inclusive state, that state follows within the
            // carry step, so the aggregate is skipped (a successor that finds
            // the flag empty waits for the inclusive state).
            if (wave == 1 && tt > 0 && s_pred_inc == 0u) {
                Cx Pt[kNPL], Ht[kNPL];
                tile_aggregate(s_aggP, s_aggH, lane, Pt, Ht);
                st_pay(mine, 0, lane, to_f2(Pt[0]), to_f2(Pt[1]));
                st_pay(mine, 1, lane, to_f2(Ht[0]), to_f2(Ht[1]));
                wait_stores();
                test_publish_delay(tc.g, tt, 1u);
                if (lane == 0) __hip_atomic_store(&flag[tt], kFlagAggregate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (has_next) issue_dma<T, DISC>(p, lay, tn, lane, wave - 1, &s_bcb[buf ^ 1][0][0], s_raw, s_k);
        } else {
            Cx Pt[kNPL], Ht[kNPL], carry[kNPL];
#pragma unroll
            for (int j = 0; j < kNPL; ++j) carry[j] = {0.f, 0.f};
            if (pred_inc) {  // the predecessor's state, loaded at the start of the tile
#pragma unroll
                for (int j = 0; j < kNPL; ++j) carry[j] = to_cx(pred_state[j]);
            }
            tile_aggregate(s_aggP, s_aggH, lane, Pt, Ht);
            // re-read the wave aggregates from LDS after the look-back rather
            // than holding them in registers across it
            asm volatile("" ::: "memory");
            if (pred_inc) {
                // carry already formed
            } else if (tt > 0) {
                look_back(flag, pay_base, tt, lane, carry);
            } else if (p.h0 || (kTR && p.q0)) {
                // the state before step 0; the trapezoid carries the shifted
                // state, g_{-1} = h_{-1} + beta'_0 q_{-1} with beta'_0 = (1 - lambda_0) delta_0
                using E = Elem<T>;
                float bp0 = 0.f;
                if constexpr (kTR) {
                    if (p.q0 && cok) {
                        const int64_t i0 = tc.b * L * D + d;
                        bp0 = (1.f - E::load(lambda, i0)) * E::load(delta, i0);
                    }
                }
#pragma unroll
                for (int j = 0; j < kNPL; ++j) {
                    if (!nok[j]) continue;
                    const int64_t hs = (tc.b * D + d) * N + pr * kNPL + j;
                    Cx g0 = {0.f, 0.f};
                    if (p.h0) g0 = CPLX ? Cx{p.h0[2 * hs], p.h0[2 * hs + 1]} : Cx{p.h0[hs], 0.f};
                    if (kTR && p.q0) {
                        const Cx q = CPLX ? Cx{p.q0[2 * hs], p.q0[2 * hs + 1]} : Cx{p.q0[hs], 0.f};
                        g0 = {g0.re + bp0 * q.re, g0.im + bp0 * q.im};
                    }
                    carry[j] = g0;
                }
            }
            // every wave's incoming state first (LDS only), then the stores
#pragma unroll
            for (int j = 0; j < kNPL; ++j) {
                Cx hin = carry[j];  // incoming state of each wave's steps
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    s_carry[w][lane][j] = to_f2(hin);
                    hin = cfma(to_cx(s_aggP[(w * 64 + lane) * kNPL + j]), hin,
                               to_cx(s_aggH[(w * 64 + lane) * kNPL + j]));
                }
            }
            Cx inc[kNPL];
#pragma unroll
            for (int j = 0; j < kNPL; ++j) inc[j] = cfma(Pt[j], carry[j], Ht[j]);
            st_pay(mine, 2, lane, to_f2(inc[0]), to_f2(inc[1]));
#pragma unroll
            for (int j = 0; j < kNPL; ++j) {
                if (tt == lay.n_tt - 1 && p.h_last && nok[j]) {
                    const int64_t hs = (tc.b * D + d) * N + pr * kNPL + j;
                    if constexpr (CPLX) {
                        p.h_last[2 * hs] = inc[j].re;
                        p.h_last[2 * hs + 1] = inc[j].im;
                    } else {
                        p.h_last[hs] = inc[j].re;
                    }
                }
            }
        }
        // Every wave, with no branch around it: the ticket after next and
        // the next tile's predecessor flag (see pred_flag), taken by lane 0 of
        // wave 0 only; every other lane's offset falls outside the window, so
        // its atomic or load does nothing (the flag then reads as empty, as it
        // does without a predecessor).  Results that are neither uniform nor
        // defined in a branch are not waited for before they are used: the
        // ticket goes to LDS at the start of the next tile, the flag is read
        // there.
        {
            const bool w0l0 = wave == 0 && lane == 0;
            ticket = static_cast<uint32_t>(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
                1, make_rsrc(&ctrl[slot], 4), w0l0 ? 0u : kOutOfRange, 0, 0));
            pred_flag = __builtin_amdgcn_raw_buffer_load_b32(
                make_rsrc(flags + tn.g * lay.n_tt, static_cast<uint32_t>(tn.tt) * 4u),
                w0l0 && tn.tt > 0 ? static_cast<uint32_t>(tn.tt - 1) * 4u : kOutOfRange, 0, kCpolSc1);
        }
        // The next tile's copies (waves 1..) and the inclusive stores (wave 0)
        // stay in flight into pass 2; the inclusive flag and the next tile's
        // register loads follow once its first outputs are out (see pass 2).
        lds_barrier();

        // ---- 4. incoming state of this wave's steps (formed by wave 0)
        Cx h[kNPL];
#pragma unroll
        for (int j = 0; j < kNPL; ++j) h[j] = to_cx(s_carry[wave][lane][j]);

        // ---- 5. pass 2: recurrence from the incoming state, outputs (y through
        // a resource covering this wave's valid steps; stores past it drop)
        {
            const int64_t yw0 = tc.t0() + s0;
            const int64_t ysteps = L - yw0 < 0 ? 0 : (L - yw0 > kTW ? kTW : L - yw0);
            const uint32_t y_row = static_cast<uint32_t>(D) * es;
            const rsrc_t rY = make_rsrc(y + (tc.b * L + (ysteps ? yw0 : 0)) * D + tc.d0,
                                        ysteps ? static_cast<uint32_t>((ysteps - 1) * D + tc.nch) * es : 0u);
            const uint32_t y_lane = cok ? static_cast<uint32_t>(c) * es : kOutOfRange;
            // the next step's LDS operands are read one step ahead
            float2 nx_dw = s_dw[s0][c];
            float4 nx_b[kNPL];
#pragma unroll
            for (int j = 0; j < kNPL; ++j) nx_b[j] = s_bc[s0][j * kLPC + pr];
#pragma unroll
            for (int s = 0; s < kTW; ++s) {
                const float2 tc4 = nx_dw;  // (delta, w)
                float4 cb[kNPL];
#pragma unroll
                for (int j = 0; j < kNPL; ++j) cb[j] = nx_b[j];
                if (s + 1 < kTW) {
                    nx_dw = s_dw[s0 + s + 1][c];
#pragma unroll
                    for (int j = 0; j < kNPL; ++j) nx_b[j] = s_bc[s0 + s + 1][j * kLPC + pr];
                }
                // Re(sum_j C h) of this lane's states as one chain of fmas
                float part;
#pragma unroll
                for (int j = 0; j < kNPL; ++j) {
                    const float4 bcq = cb[j];
                    if constexpr (CPLX) {
                        h[j] = cfma(Cx{al_r[s][j], al_i[s][j]}, h[j], Cx{tc4.y * bcq.x, tc4.y * bcq.y});
                        part = j ? __builtin_fmaf(bcq.z, h[j].re, part) : bcq.z * h[j].re;
                        part = __builtin_fmaf(-bcq.w, h[j].im, part);
                    } else {
                        h[j].re = al_r[s][j] * h[j].re + al_i[s][j];
                        part = j ? __builtin_fmaf(bcq.z, h[j].re, part) : bcq.z * h[j].re;
                    }
                }
                s_red[(wave * 8 + (s & 7)) * kRedRow + lane] = part;
                if ((s & 7) == 7) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    const int sb = s - 7 + pr;  // step this lane finishes
                    const float4 v0 = *reinterpret_cast<const float4*>(&s_red[(wave * 8 + pr) * kRedRow + c * kLPC]);
                    const float4 v1 = *reinterpret_cast<const float4*>(&s_red[(wave * 8 + pr) * kRedRow + c * kLPC + 4]);
                    const float yv =
                        ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)) + s_e[s0 + sb][c];
                    BE::store(rY, y_lane + static_cast<uint32_t>(sb) * y_row, yv);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
                if (s == kOwnIssueStep) {
                    // Everything this wave issued before the output store just
                    // above has completed (the wait is normally already
                    // satisfied: the partial reads above wait for the copies
                    // into LDS).  Wave 0 raises the inclusive flag; every wave
                    // issues its register loads of the next tile, which land
                    // during the rest of the pass.
                    wait_vm_below<1>();
                    if (wave == 0) {
                        test_publish_delay(tc.g, tt, 2u);
                        if (lane == 0)
                            __hip_atomic_store(&flag[tt], kFlagInclusive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (has_next) issue_own<T, CPLX>(r, p, tn, tid, c, pr, s0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();  // LDS is rewritten by the next tile
        if (!has_next) break;
        tc = tn;
        buf ^= 1;
    }
}

// Resident workgroups of `kernel` per CU, queried once per instantiation.
template <typename K>
int chunk_blocks_per_cu(K kernel) {
    static int cached = 0;
    if (cached == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, chunk::kThreads, 0) != hipSuccess || n < 1) n = 1;
        cached = n;
    }
    return cached;
}

template <typename T, int DISC, bool CPLX>
hipError_t launch_chunk_pair(const ChunkParams& p, const ChunkLayout& lay, dim3 pgrid, hipStream_t s) {
    using namespace chunk;
    auto kernel = chunk_scan_kernel<T, DISC, CPLX>;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t resident = int64_t(chunk_blocks_per_cu(kernel)) * cus;
    int64_t grid = int64_t(kSlots) * lay.max_slot_tiles;
    const int64_t cap = (resident / kSlots) * kSlots;
    if (cap >= kSlots && grid > cap) grid = cap;
    hipLaunchKernelGGL((chunk_prep_kernel<T, CPLX, DISC == kTrap>), pgrid, dim3(256), 0, s, p, lay);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, p, lay);
    return hipGetLastError();
}

// ---------------------------------------------------------------- launch

template <typename T>
int launch_chunked(int disc, bool cplx, const ChunkParams& p, hipStream_t s) {
    using namespace chunk;
    const ChunkLayout lay = chunk_layout(p.batch, p.seqlen, p.dim);
    if (int64_t(kSlots) * lay.max_slot_tiles > UINT32_MAX || lay.groups > INT32_MAX)
        return 2;  // SSM_ERR_UNSUPPORTED: tickets and group indices are 32-bit
    // buffer windows and per-lane byte offsets are 32-bit: keep every window
    // (and an out-of-range lane offset plus a window) below 2^31
    const uint64_t es = sizeof(T), lim = uint64_t(1) << 30;
    if (uint64_t(p.dim) * p.dstate * es * kTW > lim || uint64_t(kTT + 2) * p.dim * es > lim ||
        uint64_t(p.dim) * p.dstate * 4 > lim)
        return 2;
    const int64_t items = p.batch * lay.l_pad * kChunkLanes;
    const int64_t nfl = lay.groups * lay.n_tt;
    int64_t pblocks = ((items > nfl ? items : nfl) + 255) / 256;
    if (pblocks > 16384) pblocks = 16384;
    const dim3 pg(static_cast<unsigned>(pblocks));
    hipError_t e;
    if (cplx) {
        e = disc == kEuler ? launch_chunk_pair<T, kEuler, true>(p, lay, pg, s)
                           : launch_chunk_pair<T, kTrap, true>(p, lay, pg, s);
    } else {
        e = disc == kZOH     ? launch_chunk_pair<T, kZOH, false>(p, lay, pg, s)
            : disc == kEuler ? launch_chunk_pair<T, kEuler, false>(p, lay, pg, s)
                             : launch_chunk_pair<T, kTrap, false>(p, lay, pg, s);
    }
    return e == hipSuccess ? 0 : -static_cast<int>(e);
}

}  // namespace ssm
