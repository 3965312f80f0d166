/*
 * ssm_scan.h -- C ABI of libssmscan.so, the forward selective scan for
 * AMD MI355X (gfx950).
 *
 * The operation (per batch b, channel d, state n; h_{-1} = 0):
 *
 *   alpha_t[n] = exp(delta_t A[d,n]) * e^{i theta_t[n]}      (complex state)
 *              = exp(delta_t A[d,n])                          (real state)
 *   h_t[n]     = alpha_t[n] h_{t-1}[n] + bterm_t[n]
 *   y_t        = Re( sum_n C_t[n] h_t[n] ) + D[d] u_t
 *
 * with the b-term of the chosen discretisation (q_t[n] = B_t[n] u_t):
 *   ZOH                  bterm = (exp(delta A) - 1)/A * q_t      (delta q_t if A = 0)
 *   exponential Euler    bterm = delta_t q_t
 *   exp.-trapezoidal     bterm = lambda_t delta_t q_t
 *                              + (1 - lambda_t) delta_t alpha_t q_{t-1},  q_{-1} = 0
 *
 * Sources: the recurrence and its associative combine follow the
 * fengwang.github.io essay on the complex parallel scan (section on the
 * mathematics of the parallel scan); the three discretisations follow the
 * discretisation table of the ai.tomabc.com Mamba-3 paper story, and its
 * complex-state section for the rotation e^{i theta_t} with A real; the ZOH
 * form also appears in section 2.1 of the blog.lonae.com essay on the dual
 * spectral theory of SSMs and section 2.2 of the metaphor-xennon Mamba-3
 * notes; the output uses the post-update state as in the mamba2_ssd loop of
 * the blog.lonae.com essay (section 3.2).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    dense row-major in the index order given, with no strides.  Complex
 *    values are interleaved (re, im).
 *  - The caller allocates and owns every buffer, including the workspace.
 *    The library allocates no device memory, keeps no pointer after the call
 *    returns, and never synchronises the host with the device.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    Buffers must stay valid until that work completes.  Faults during
 *    execution surface at the caller's next synchronisation of the stream.
 *  - Outputs must not alias inputs.  Calls that share a workspace must not
 *    overlap in time (they would race on its flags).
 *  - Every argument is validated before any HIP call; an invalid call
 *    returns a non-zero status and enqueues nothing.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 5

/* Element type of u, delta, B, C, theta, lambda and y.  A, D and h_last are
 * always fp32; all arithmetic is fp32 (bf16 inputs are widened exactly, y is
 * rounded to nearest-even on the way out). */
typedef enum { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype_t;

typedef enum {
    SSM_DISC_ZOH = 0,             /* real state only */
    SSM_DISC_EXP_EULER = 1,
    SSM_DISC_EXP_TRAPEZOIDAL = 2  /* needs lambda */
} ssm_disc_t;

/* Kernel family.  SEQUENTIAL sweeps the whole sequence per channel (one
 * channel's states across lanes; needs many channels to fill the GPU; any
 * N <= 64).  CHUNKED splits the sequence into tiles of 96 steps x 8 channels,
 * keeps each tile's state in registers and carries it between tiles with a
 * decoupled look-back (fills the GPU at any shape; N <= 16).  SWEEP gives
 * each lane one (channel, state) and sweeps the whole sequence in one pass,
 * 16 steps at a time staged through LDS (N <= 16; needs no workspace; fills
 * the GPU once B * ceil(D/4) reaches a few waves per SIMD; UNSUPPORTED when
 * 34*D*N*esize reaches 2^31).  AUTO uses SWEEP when N <= 16 and either
 * L <= 96 or B * ceil(D/4) reaches 1536 for a real state, 2048 for a complex
 * exp-Euler one or 3072 for the complex trapezoid (1.5, 2 and 3 waves per
 * SIMD of a 256-CU GPU, where it measured faster), else CHUNKED when
 * N <= 16, else SEQUENTIAL.  All give the same result up to rounding. */
typedef enum {
    SSM_ALGO_AUTO = 0,
    SSM_ALGO_SEQUENTIAL = 1,
    SSM_ALGO_CHUNKED = 2,
    SSM_ALGO_SWEEP = 3
} ssm_algo_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARGUMENT = 1,   /* null required pointer, bad size, overflow,
                                       misalignment, forbidden NULL/non-NULL combination */
    SSM_ERR_UNSUPPORTED = 2,        /* complex ZOH, dstate > 64 (> 16 for CHUNKED and SWEEP),
                                       unknown enum value, or (CHUNKED) a shape whose
                                       per-tile windows exceed 32-bit offsets:
                                       24*D*N*esize, 98*D*esize or 4*D*N above 2^30 */
    SSM_ERR_WORKSPACE_TOO_SMALL = 3,
    SSM_ERR_HIP = 4,                /* a HIP call failed; see ssm_scan_last_hip_error() */
    SSM_ERR_SCRATCH_LIMIT = 5       /* ssm_scan_fwd_noalloc: the problem needs more scratch
                                       than SSM_SCAN_NOALLOC_SCRATCH_BYTES */
} ssm_status_t;

typedef struct {
    int64_t batch;   /* B >= 1 */
    int64_t seqlen;  /* L >= 1 */
    int64_t dim;     /* D >= 1, channels */
    int64_t dstate;  /* N, 1 <= N <= 64 */
    int32_t io_dtype;   /* ssm_dtype_t */
    int32_t disc;       /* ssm_disc_t */
    int32_t is_complex; /* 0: real state, B, C real; 1: complex state, B, C complex */
    int32_t algo;       /* ssm_algo_t */
} ssm_scan_desc_t;

/* Bytes of workspace ssm_scan_fwd needs for `desc` (0 when the chosen kernel
 * needs none).  Returns 0 for an invalid descriptor as well; ssm_scan_fwd
 * reports that case.  For CHUNKED it is about 3 KiB per tile (96 steps x 8
 * channels: the look-back payloads) plus 260 bytes per (batch, step) for the
 * fp32 B/C rows; e.g. 4.6 GB for B=1, L=2^20, D=1024. */
size_t ssm_scan_workspace_bytes(const ssm_scan_desc_t *desc);

/* The kernel family ssm_scan_fwd runs for `desc` (an ssm_algo_t other than
 * SSM_ALGO_AUTO: desc->algo itself when it is not AUTO, else the family AUTO
 * picks for the shape), or -1 for an invalid descriptor.  Touches no device. */
int ssm_scan_algo(const ssm_scan_desc_t *desc);

/*
 * Forward selective scan.
 *
 *   u       [B][L][D]          io dtype   input x_t of each channel
 *   delta   [B][L][D]          io dtype   step sizes Delta_t (> 0 expected, not checked)
 *   A       [D][N]             fp32       diagonal state matrix (real)
 *   B       [B][L][N]          io dtype   real input projection, or
 *           [B][L][N][2]                  complex (is_complex = 1)
 *   C       same layout as B              output projection (no conjugate)
 *   D       [D] fp32 or NULL              skip term; NULL means 0
 *   theta   [B][L][D][N] io dtype or NULL rotation angle (radians) of the complex
 *                                         state; must be NULL when is_complex = 0;
 *                                         NULL with is_complex = 1 means theta = 0
 *   lambda  [B][L][D] io dtype            trapezoid weight; required for
 *                                         EXP_TRAPEZOIDAL, must be NULL otherwise
 *   y       [B][L][D] io dtype            output (written)
 *   h_last  [B][D][N] fp32, or            final state h_{L-1} (written);
 *           [B][D][N][2], or NULL         NULL means not written
 *   workspace, workspace_bytes            device scratch of at least
 *                                         ssm_scan_workspace_bytes(desc) bytes,
 *                                         256-byte aligned; may be NULL when that
 *                                         is 0.  Its contents need no
 *                                         initialisation and are not preserved.
 *   stream                                hipStream_t (NULL = default stream)
 *
 * Alignment: every pointer must be aligned to its element size (4 bytes for
 * fp32, 2 for bf16, 8 for complex fp32 h_last).  CHUNKED stages u, delta and
 * lambda by 16-byte DMA when D * element size is a multiple of 16 and those
 * pointers are 16-byte aligned; other shapes take a slower element-wise
 * staging path with the same results.  Returns an ssm_status_t.
 */
int ssm_scan_fwd(const ssm_scan_desc_t *desc, const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *theta,
                 const void *lambda, void *y, float *h_last, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * Continuation of a scan: the same operation over a sequence that began
 * before step 0.  A long sequence can be processed in pieces, or a prompt
 * scanned and its state handed to ssm_scan_step for decoding.  The state is
 * the whole memory a recurrent model carries, so a state left by one call
 * serves as the prefix of the next (the production
 * checklist of the blog.lonae.com essay, on reusing the state; the
 * ai.tomabc.com Mamba-3 story's motivation section, on the fixed-size state
 * of recurrent inference).  Arguments as for ssm_scan_fwd, plus:
 *
 *   h0      [B][D][N] fp32, or [B][D][N][2]    state before step 0 (h_{-1});
 *           (is_complex = 1), or NULL            NULL means 0
 *   q0      same layout as h0, or NULL          q_{-1} = B_{-1} u_{-1}, the input
 *                                               term of the step before step 0,
 *                                               which the trapezoid's beta_0
 *                                               multiplies; EXP_TRAPEZOIDAL only
 *                                               (must be NULL otherwise); NULL means 0
 *   q_last  same layout as h0, or NULL          q_{L-1} = B_{L-1} u_{L-1} (written);
 *                                               EXP_TRAPEZOIDAL only
 *
 * Passing h_last and q_last of one call as h0 and q0 of the next gives the
 * result of a single call over the concatenated sequence (up to rounding).
 * h0 and q0 must not alias h_last, q_last or any other output.  Each state
 * pointer must be aligned to one state element (8 bytes complex, 4 real).
 * ssm_scan_fwd is this call with h0, q0 and q_last NULL.  Returns an
 * ssm_status_t.
 */
int ssm_scan_fwd_ex(const ssm_scan_desc_t *desc, const void *u, const void *delta, const float *A,
                    const void *B, const void *C, const float *D, const void *theta,
                    const void *lambda, const float *h0, const float *q0, void *y, float *h_last,
                    float *q_last, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the fixed per-GPU scratch buffer of ssm_scan_fwd_noalloc. */
#define SSM_SCAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, results and errors are those of ssm_scan_fwd, except that there
 * is no workspace argument: the kernels use a fixed scratch buffer of
 * SSM_SCAN_NOALLOC_SCRATCH_BYTES inside the library instead, one per GPU,
 * which exists from the loading of the library's code on that GPU until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or other
 * allocating routine).
 *
 *  - Limit: when ssm_scan_workspace_bytes(desc) exceeds
 *    SSM_SCAN_NOALLOC_SCRATCH_BYTES the call returns SSM_ERR_SCRATCH_LIMIT
 *    before any HIP call; such problems need ssm_scan_fwd with a workspace.
 *  - Device: the buffer of the current HIP device is used, so `stream` must
 *    belong to it.  The first call on a device looks up that device's buffer
 *    address; if that lookup fails the call returns SSM_ERR_HIP.
 *  - Sharing: every call on one GPU uses that GPU's buffer, and the buffer
 *    keeps the last call's contents.  Each call re-initialises on its stream,
 *    with a kernel (no memset), everything the kernels need to start at zero.
 *    Calls on one GPU must not overlap in time: they would race on the buffer.
 */
int ssm_scan_fwd_noalloc(const ssm_scan_desc_t *desc, const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *theta,
                         const void *lambda, void *y, float *h_last, void *stream);

/*
 * One step of the recurrence with the state kept in device memory and
 * updated in place: the decode step of autoregressive generation, where each
 * new token advances the fixed-size state once (the ai.tomabc.com Mamba-3
 * story's table of inference arithmetic intensity treats this sequential
 * step; it reads and writes the whole state per token, so it is bound by
 * memory traffic).  desc->seqlen must be 1; desc->algo is ignored.  The
 * tensors are those of ssm_scan_fwd with the length-1 time axis dropped:
 *
 *   u, delta, lambda  [B][D] io dtype     inputs of this step (lambda: EXP_TRAPEZOIDAL
 *                                         only, NULL otherwise)
 *   A [D][N] fp32, D [D] fp32 or NULL     as for ssm_scan_fwd
 *   B, C   [B][N] or [B][N][2] io dtype   projections of this step
 *   theta  [B][D][N] io dtype or NULL     rotation of this step (complex state)
 *   u_prev [B][D] io dtype, or NULL       EXP_TRAPEZOIDAL: u and B of the previous
 *   B_prev layout of B, or NULL           step, whose product q_{t-1} = B_{t-1} u_{t-1}
 *                                         the trapezoid's beta multiplies; both NULL
 *                                         means no previous step (q_{t-1} = 0);
 *                                         must be NULL for the other discretisations
 *   h      [B][D][N] or [B][D][N][2] fp32 read as h_{t-1}, overwritten with h_t
 *                                         (required)
 *   y      [B][D] io dtype                output of this step (written)
 *
 * After a prompt scanned by ssm_scan_fwd_ex, its h_last is the state and the
 * prompt's last u and B rows are u_prev and B_prev.  N may be up to 64.  No
 * workspace.  h must not alias any other argument.  Returns an ssm_status_t.
 */
int ssm_scan_step(const ssm_scan_desc_t *desc, const void *u, const void *delta, const float *A,
                  const void *B, const void *C, const float *D, const void *theta, const void *lambda,
                  const void *u_prev, const void *B_prev, float *h, void *y, void *stream);

/* Bytes of workspace ssm_scan_bwd needs for `desc`: the state before every
 * 8-step segment, ceil(L/8) * B * D * N * (8 complex, 4 real) bytes
 * (e.g. 1.34 GB for B=4, L=8192, D=2560, N=16 complex), rounded up to 256,
 * plus, when the sequence is cut into time chunks (problems with fewer than
 * about 2^19 (channel, state) lanes, chunks of at least 256 steps), one
 * adjoint pair per chunk and (b, d, n): chunks * B * D * N * (16 complex,
 * 8 real) bytes.  0 for an invalid descriptor. */
size_t ssm_scan_bwd_workspace_bytes(const ssm_scan_desc_t *desc);

/*
 * Gradients of the scan (the backward pass), for
 *     Loss = sum(dy * y) + <dh_last, h_last>
 * with y, h_last the outputs of ssm_scan_fwd_ex(..., h0, q0 = NULL, ...) on the
 * same inputs.  The forward states are regenerated from per-segment
 * snapshots during the reverse sweep and never stored whole, which is how
 * the fengwang.github.io essay describes training a scan (its opening
 * section, and its hardware-challenges section on the backward kernel with
 * recomputation); the gradient formulas are reverse-mode differentiation of
 * the recurrence and discretisations above.
 *
 *   inputs   u, delta, A, B, C, D, theta, lambda, h0 as for ssm_scan_fwd_ex
 *            (h0 may be NULL; desc->algo is ignored)
 *   dy       [B][L][D] io dtype        upstream gradient of y
 *   dh_last  layout of h_last, or NULL upstream gradient of h_last (NULL: 0)
 * outputs (fp32, written; complex gradients are (dL/dRe, dL/dIm)):
 *   du, ddelta        [B][L][D]                   required
 *   dA                [D][N]                      required (sum over b, t)
 *   dB, dC            layout of B and C           required (sum over d)
 *   dD                [D], or NULL                sum over b, t of dy * u
 *   dtheta            [B][L][D][N], or NULL       only when theta is given
 *   dlambda           [B][L][D]                   required for EXP_TRAPEZOIDAL,
 *                                                 NULL otherwise
 *   dh0               layout of h_last, or NULL   gradient of the state before step 0
 *   workspace         ssm_scan_bwd_workspace_bytes(desc) bytes, 256-byte aligned
 *
 * dA, dB, dC and dD are sums taken with atomic adds, so their last bits can
 * vary between runs.  Outputs must not alias inputs or each other.  Returns
 * an ssm_status_t.
 */
int ssm_scan_bwd(const ssm_scan_desc_t *desc, const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *theta, const void *lambda,
                 const float *h0, const void *dy, const float *dh_last, float *du, float *ddelta,
                 float *dA, float *dB, float *dC, float *dD, float *dtheta, float *dlambda, float *dh0,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * The state-space dual (SSD) form, for heads with a scalar decay
 * (blog.lonae.com essay on the dual spectral theory of SSMs, section 3,
 * "Mamba-2's SSD duality"): the channels of a head share delta_t and a
 * scalar A, so all their states decay alike, and the scan becomes a causal
 * decaying linear attention computed chunk by chunk with matrix products.
 * For channel d of head h = d / headdim, with exponential-Euler b-terms:
 *
 *   h_t[n] = exp(delta_t[h] A[h]) h_{t-1}[n] + delta_t[h] B_t[n] u_t[d],   h_{-1} = 0
 *   y_t[d] = sum_n C_t[n] h_t[n] + D[d] u_t[d]
 *
 * which is ssm_scan_fwd (real state, EXP_EULER) with delta and A broadcast
 * over each head's channels.
 */
typedef struct {
    int64_t batch;    /* B >= 1 */
    int64_t seqlen;   /* L >= 1 */
    int64_t dim;      /* D >= 1, a multiple of headdim */
    int64_t dstate;   /* N, 1 <= N <= 64 */
    int64_t headdim;  /* channels per head; 64 */
    int32_t io_dtype; /* SSM_DTYPE_BF16 (fp32 I/O returns SSM_ERR_UNSUPPORTED) */
    int32_t reserved; /* 0 */
} ssm_ssd_desc_t;

/* Bytes of workspace ssm_ssd_fwd needs: two bf16 N x headdim states and one
 * fp32 decay per (batch, head, 64-step chunk); 0 for an invalid or
 * unsupported descriptor. */
size_t ssm_ssd_workspace_bytes(const ssm_ssd_desc_t *desc);

/*
 *   u       [B][L][D]   bf16     inputs (16-byte aligned: read in rows of 8 channels)
 *   delta   [B][L][H]   bf16     step size of each head (H = D / headdim)
 *   A       [H]         fp32     scalar decay rate of each head
 *   B, C    [B][L][N]   bf16     projections shared by all heads
 *   D       [D] fp32 or NULL     skip term
 *   y       [B][L][D]   bf16     output (written; 16-byte aligned like u)
 *   h_last  [B][D][N] fp32, or NULL   final state (written)
 *   workspace  ssm_ssd_workspace_bytes(desc) bytes, 256-byte aligned
 * Returns an ssm_status_t (SSM_ERR_UNSUPPORTED for fp32 I/O, headdim != 64,
 * D not a multiple of headdim or N > 64).
 */
int ssm_ssd_fwd(const ssm_ssd_desc_t *desc, const void *u, const void *delta, const float *A,
                const void *B, const void *C, const float *D, void *y, float *h_last, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * The multi-input multi-output (MIMO) scan: each (b, d) channel keeps ONE
 * state h[n] that R inputs feed and R outputs read.  B and C are N x R per
 * step instead of N-vectors (the ai.tomabc.com Mamba-3 story, MIMO section
 * and its shape table: R parallel input/output channels share the state,
 * and the work per step grows from O(N) to O(N R) with the same state
 * traffic; the metaphor-xennon Mamba-3 notes, section 3.3).  Per b, d, n:
 *
 *   q_t[n] = sum_r B_t[n, r] u_t[r]
 *   h_t[n] = alpha_t[n] h_{t-1}[n] + bterm_t[n]     (alpha and bterm of the
 *            chosen discretisation exactly as for ssm_scan_fwd, with this
 *            q_t; the trapezoid's q_{t-1} is the previous step's sum)
 *   y_t[r] = Re( sum_n C_t[n, r] h_t[n] ) + D[d] u_t[r]
 *
 * R = 1 is ssm_scan_fwd_ex with a trailing unit axis on u, B, C and y.
 */
typedef struct {
    int64_t batch;      /* B >= 1 */
    int64_t seqlen;     /* L >= 1 (1 for ssm_mimo_step) */
    int64_t dim;        /* D >= 1 */
    int64_t dstate;     /* N, 1 <= N <= 64 */
    int64_t rank;       /* R: inputs and outputs per token and channel; 1, 2, 4 or 8 */
    int64_t chunk;      /* steps per time chunk; 0 lets the library choose (ignored by the step) */
    int32_t io_dtype;   /* ssm_dtype_t */
    int32_t disc;       /* ssm_disc_t */
    int32_t is_complex; /* 0 or 1, as for ssm_scan_desc_t */
    int32_t reserved;   /* 0 */
} ssm_mimo_desc_t;

/* Bytes of workspace ssm_mimo_fwd needs: a (decay product, state) pair per
 * (b, d, n) for every time chunk but the last, (chunks - 1) * B * D * N *
 * (16 complex, 8 real) bytes; 0 when one chunk covers the sequence or the
 * descriptor is invalid.  The library's choice of chunk depends only on the
 * descriptor. */
size_t ssm_mimo_workspace_bytes(const ssm_mimo_desc_t *desc);

/*
 *   u       [B][L][D][R]   io dtype   inputs (aligned to min(16, R * element) bytes)
 *   delta, lambda  [B][L][D] io dtype as for ssm_scan_fwd (lambda: EXP_TRAPEZOIDAL only)
 *   A [D][N] fp32, D [D] fp32 or NULL as for ssm_scan_fwd; D is shared by a channel's R outputs
 *   B, C    [B][L][N][R] or [B][L][N][R][2] io dtype
 *                                     (aligned to min(16, R * 2 * element) bytes if complex,
 *                                     min(16, R * element) if real)
 *   theta   [B][L][D][N] io dtype or NULL   as for ssm_scan_fwd
 *   h0, q0, h_last, q_last            as for ssm_scan_fwd_ex, with q = the sum above
 *   y       [B][L][D][R]   io dtype   output (written; aligned like u)
 *   workspace  ssm_mimo_workspace_bytes(desc) bytes, 16-byte aligned (may be
 *              NULL when that is 0)
 * Returns an ssm_status_t (SSM_ERR_UNSUPPORTED for R not in {1, 2, 4, 8},
 * N > 64 or complex ZOH).
 */
int ssm_mimo_fwd(const ssm_mimo_desc_t *desc, const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *theta, const void *lambda,
                 const float *h0, const float *q0, void *y, float *h_last, float *q_last, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * One decode step of the MIMO recurrence, the state kept by the caller
 * (the regime of the Mamba-3 story's inference table: R times the work of
 * the single-input step for the same state traffic).  desc->seqlen must be
 * 1.  The tensors are those of ssm_mimo_fwd with the time axis dropped:
 *   u [B][D][R], delta and lambda [B][D], B and C [B][N][R] (or [..][2]),
 *   theta [B][D][N] or NULL, y [B][D][R];
 *   u_prev [B][D][R] and B_prev (layout of B): EXP_TRAPEZOIDAL only, the
 *   previous step's inputs whose sum q_{t-1} the trapezoid's beta multiplies;
 *   both NULL means no previous step;
 *   h  [B][D][N] or [B][D][N][2] fp32, read as h_{t-1} and overwritten with h_t.
 * Alignment as for ssm_mimo_fwd.  Returns an ssm_status_t.
 */
int ssm_mimo_step(const ssm_mimo_desc_t *desc, const void *u, const void *delta, const float *A,
                  const void *B, const void *C, const float *D, const void *theta, const void *lambda,
                  const void *u_prev, const void *B_prev, float *h, void *y, void *stream);

/* Static description of a status code (never NULL). */
const char *ssm_scan_status_string(int status);

/* The hipError_t of the last failed HIP call made by this thread inside the
 * library (0 if none). */
int ssm_scan_last_hip_error(void);

/* SSM_SCAN_ABI_VERSION of the loaded library. */
int ssm_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
