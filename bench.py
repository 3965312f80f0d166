#!/usr/bin/env python3
"""Throughput of the forward selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--algo auto]

A step is one full scan (discretisation, recurrence, output contraction,
carry between tiles) over one batch of seeded synthetic inputs that are
already resident in HBM.  Rank 0 prints one JSON line:

  value      tokens*channels/s = B*L*D / (seconds per step)
  roofline   algorithmic HBM bytes per launch / kernel time vs 8.0 TB/s
             (algorithmic bytes: every input read once, every output written
             once); `traffic` comes from the committed
             rocprofv3 counter summary when it was taken on the current
             kernel sources, else null
  cpu_baseline  the fp64 oracle timed on the host's cores over a bounded
             sample of channels of the same workload

The default workload is the largest one (B=1, D=1024, L=2^20, N=16, complex
exp-trapezoidal, bf16 I/O, fp32 arithmetic), on which the HBM-bandwidth target
is stated.  A decode workload (--workload decode_...) times ssm_scan_step
instead: a step is one token for every sequence of the batch, the state read
and written in HBM, and the same line is printed with B*D tokens*channels per
step.  --backward times ssm_scan_bwd (all input gradients of the scan) on the
workload instead of the forward scan.  An SSD workload (--workload ssd_...)
times ssm_ssd_fwd, the chunked matrix form for heads with a scalar decay.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan tokens*channels/s + achieved HBM GB/s (% of MI355X peak)"
UNIT = "tokens*channels/s"
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "complex_trap_bf16_b1_d1024_l1048576_n16"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> int:
    """Each input read once and each output written once."""
    e = 4 if w.io_dtype == "f32" else 2
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    trap = 1 if w.disc == "trap" else 0
    cplx = 1 if w.is_complex else 0
    return (e * B * L * D * (3 + trap)          # u, delta, (lambda), y
            + e * B * L * D * N * cplx          # theta
            + 2 * e * B * L * N * (1 + cplx)    # B, C
            + 4 * D * N + 4 * D                 # A, D
            + 4 * B * D * N * (1 + cplx))       # h_last


def decode_algorithmic_bytes(w) -> int:
    """One decode step: inputs of the step and the previous step's u and B rows
    read once, the state read and written once, y written once."""
    e = 4 if w.io_dtype == "f32" else 2
    B, D, N = w.batch, w.dim, w.dstate
    trap = 1 if w.disc == "trap" else 0
    cplx = 1 if w.is_complex else 0
    return (e * B * D * (3 + 2 * trap)           # u, delta, y, (lambda, u_prev)
            + e * B * D * N * cplx               # theta
            + e * B * N * (1 + cplx) * (2 + trap)  # B, C, (B_prev)
            + 4 * D * N + 4 * D                  # A, D
            + 2 * 4 * B * D * N * (1 + cplx))    # h read and written


def backward_algorithmic_bytes(w) -> int:
    """The backward pass: every input and dy read once, every gradient (fp32)
    written once."""
    e = 4 if w.io_dtype == "f32" else 2
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    trap = 1 if w.disc == "trap" else 0
    cplx = 1 if w.is_complex else 0
    reads = (e * B * L * D * (3 + trap) + e * B * L * D * N * cplx + 2 * e * B * L * N * (1 + cplx)
             + 4 * D * N + 4 * D)
    writes = (4 * B * L * D * (2 + trap) + 4 * B * L * D * N * cplx + 2 * 4 * B * L * N * (1 + cplx)
              + 4 * D * N + 4 * D)
    return reads + writes


def ssd_algorithmic_bytes(w) -> int:
    """The SSD form: u, delta (per head), B, C, A, D read once; y, h_last written once."""
    e = 2
    B, L, D, N, H = w.batch, w.seqlen, w.dim, w.dstate, w.heads
    return e * B * L * D * 2 + e * B * L * H + 2 * e * B * L * N + 4 * H + 4 * D + 4 * B * D * N


def mimo_algorithmic_bytes(w) -> int:
    """The MIMO scan: u and y (R per token and channel), delta, lambda, theta,
    B and C (N x R per step), A, D read or written once, h_last written once."""
    e = 4 if w.io_dtype == "f32" else 2
    B, L, D, N, R = w.batch, w.seqlen, w.dim, w.dstate, w.rank
    trap = 1 if w.disc == "trap" else 0
    cplx = 1 if w.is_complex else 0
    return (e * B * L * D * (2 * R + 1 + trap) + e * B * L * D * N * cplx + 2 * e * B * L * N * R * (1 + cplx)
            + 4 * D * N + 4 * D + 4 * B * D * N * (1 + cplx))


PEAK_BF16_MFMA_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
PEAK_FP32_VECTOR_TFLOPS = 157.3  # published fp32 vector peak (packed FMA: 2 lanes x 2 flops per lane-slot)


def ssd_algorithmic_flops(w, q: int = 64) -> int:
    """The SSD form's four dense products per (batch row, head, chunk of q
    steps), N states, P channels per head: C B^T (2 q^2 N), the causal
    intra-chunk product (q (q + 1) P: row t sums t + 1 terms), C H_in (2 q N P)
    and the chunk state B^T X (2 q N P)."""
    B, L, N, P, H = w.batch, w.seqlen, w.dstate, w.headdim, w.heads
    chunks = (L + q - 1) // q
    return B * H * chunks * (2 * q * q * N + q * (q + 1) * P + 4 * q * N * P)


def mimo_algorithmic_flops(w) -> int:
    """fp32 vector flops per (b, t, d, n) of the complex MIMO recurrence of
    rank R: the rotation-decay product alpha g (6) and the weighted input
    added (4), the input q = sum_r B_r u_r (4 R: a complex-by-real multiply and
    add per r) and the R outputs' Re(C_r g) (4 R).  Transcendentals are not
    counted."""
    B, L, D, N, R = w.batch, w.seqlen, w.dim, w.dstate, w.rank
    per = (10 + 8 * R) if w.is_complex else (2 + 4 * R)
    return B * L * D * N * per


def mimo_decode_algorithmic_bytes(w) -> int:
    """One MIMO decode step: the step's inputs and the previous step's u and B
    read once, the state read and written once, the R outputs written once."""
    e = 4 if w.io_dtype == "f32" else 2
    B, D, N, R = w.batch, w.dim, w.dstate, w.rank
    trap = 1 if w.disc == "trap" else 0
    cplx = 1 if w.is_complex else 0
    return (e * B * D * (2 * R + 1 + trap * (1 + R))     # u, y, delta, (lambda, u_prev)
            + e * B * D * N * cplx                        # theta
            + e * B * N * R * (1 + cplx) * (2 + trap)     # B, C, (B_prev)
            + 4 * D * N + 4 * D                           # A, D
            + 2 * 4 * B * D * N * (1 + cplx))             # h read and written


# The device code behind each path, for telling whether committed counters
# still describe the kernels that run.
KERNEL_SOURCES = {
    "chunked": ["kernel_chunked.h"],
    "sequential": ["kernel_sequential.h"],
    "sweep": ["kernel_sweep.h"],
    "step": ["kernel_step.h"],
    "backward": ["kernel_backward.h"],
    "ssd": ["kernel_ssd.h"],
    "mimo": ["kernel_mimo.h", "mimo_launch.h", "mimo.hip"],
    "mimo_step": ["kernel_mimo.h", "mimo_launch.h", "mimo.hip"],
}


def kernel_source_hash(algo: str) -> str:
    """Hash of the device sources of one path (its kernel header and the shared
    device helpers)."""
    csrc = os.path.join(ROOT, "selective_state_space_42_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[algo] + ["device_common.h", "device_math.h"]):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, algo: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(workload, {}).get(algo)
    if not entry or entry.get("source_hash") != kernel_source_hash(algo):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(inputs, w, y_gpu, target_s: float):
    """Time the fp64 oracle on a bounded channel sample; also report its parity.

    Channels are taken in groups of one per host thread (spread evenly over D)
    until about `target_s` seconds of oracle time are spent, so the host
    memory for the fp64 copy stays bounded.  Only the oracle calls are timed.
    """
    import numpy as np
    import torch

    import oracle
    from selective_state_space_42_amd.inputs import channel_sample

    threads = max(1, min(os.cpu_count() or 1, 64))
    order = np.random.default_rng(0).permutation(w.dim).tolist()
    spent, tc, used, err, groups = 0.0, 0, 0, 0.0, 0
    for g0 in range(0, w.dim, threads):
        idx = sorted(order[g0:g0 + threads])
        x = channel_sample(inputs, idx)
        t0 = time.perf_counter()
        y_ref, _ = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                               disc=w.disc, is_complex=w.is_complex, nthreads=len(idx))
        spent += time.perf_counter() - t0
        tc += w.batch * w.seqlen * len(idx)
        used = max(used, len(idx))
        groups += 1
        yg = y_gpu.index_select(2, torch.as_tensor(idx, device=y_gpu.device)).float().cpu().double().numpy()
        err = max(err, float(np.max(np.abs(yg - y_ref)) / np.max(np.abs(y_ref))))
        del x, y_ref, yg
        if spent >= target_s:
            break
    return {
        "value": tc / spent, "unit": UNIT, "cores": used, "kind": "oracle",
        "sample": f"{tc // (w.batch * w.seqlen)} of {w.dim} channels (random, seed 0) in {groups} group(s), "
                  f"every batch row and step, N={w.dstate}: {tc} tokens*channels in {spent:.1f} s of "
                  f"fp64 C oracle time on {used} pthreads",
        "parity_err_y_on_sample": err,
    }


def cpu_baseline_decode(inputs, w, h_start, target_s: float):
    """Time the fp64 oracle on one decode step of a channel sample (the oracle
    run for one step from the given state), repeated up to `target_s` s."""
    import numpy as np

    import oracle
    from selective_state_space_42_amd.inputs import channel_sample

    threads = max(1, min(os.cpu_count() or 1, 64))
    idx = sorted(np.random.default_rng(0).permutation(w.dim)[:max(threads, 64)].tolist())
    x = channel_sample(inputs, idx)
    cur = {k: (None if v is None else (v[:, 1:2] if k in ("u", "delta", "lam", "theta", "Bm", "Cm") else v))
           for k, v in x.items()}
    h0 = h_start[:, idx].float().cpu().double().numpy()
    q0 = None
    if w.disc == "trap":  # q_{-1} = B_{-1} u_{-1}, previous step's rows
        bp, up = x["Bm"][:, 0], x["u"][:, 0]
        q0 = (bp[:, None, ...] * (up[:, :, None, None] if w.is_complex else up[:, :, None]))
    spent, calls = 0.0, 0
    while spent < target_s:
        t0 = time.perf_counter()
        oracle.scan(cur["u"], cur["delta"], cur["A"], cur["Bm"], cur["Cm"], cur["Dskip"], cur["theta"],
                    cur["lam"], disc=w.disc, is_complex=w.is_complex, h0=h0, q0=q0, nthreads=threads)
        spent += time.perf_counter() - t0
        calls += 1
    tc = calls * w.batch * len(idx)
    return {
        "value": tc / spent, "unit": UNIT, "cores": min(threads, len(idx)), "kind": "oracle",
        "sample": f"{len(idx)} of {w.dim} channels (random, seed 0), every batch row, one decode step from a "
                  f"given state, repeated {calls} times: {tc} tokens*channels in {spent:.1f} s of fp64 C "
                  f"oracle time",
    }


EVICT_BYTES = 1 << 30  # scratch written before every timed rep: evicts the L2s and the 256 MB MALL


class Timing:
    """Per-rep times (ms) of a timed loop; `ms` (the median) is what a step costs."""

    def __init__(self, reps):
        self.reps = sorted(reps)
        n = len(self.reps)
        self.median = self.reps[n // 2] if n % 2 else 0.5 * (self.reps[n // 2 - 1] + self.reps[n // 2])
        self.min = self.reps[0]
        self.mean = sum(self.reps) / n

    @property
    def ms(self):
        return self.median

    def record(self):
        return {"median_ms": self.median, "min_ms": self.min, "mean_ms": self.mean, "reps": len(self.reps),
                "method": "HIP events around each step on the launch stream; before every step a "
                          f"{EVICT_BYTES >> 20} MiB scratch buffer is written outside the events (L2/MALL eviction)"}


def _timed(torch, stream, step, steps: int, warmup: int, label: str = "steps") -> Timing:
    """Warm up, then time each of `steps` calls of step() with its own event
    pair on `stream`, writing a 1 GiB scratch buffer before each call (outside
    the events) so that no input is served from the L2s or the MALL."""
    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{warmup} done")
    scratch = torch.empty(EVICT_BYTES // 4, dtype=torch.float32, device=torch.cuda.current_device())
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(events):
            scratch.fill_(float(i))
            a.record(stream)
            step()
            b.record(stream)
    torch.cuda.synchronize()
    t = Timing([a.elapsed_time(b) for a, b in events])
    del scratch
    log(f"timed {steps} {label}: median {t.median:.4f} ms, min {t.min:.4f} ms, mean {t.mean:.4f} ms")
    return t


def bench_decode(args, w, torch, dev):
    from selective_state_space_42_amd.inputs import make_inputs
    from selective_state_space_42_amd.scan import ssm_scan_step

    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_inputs(w, device=dev)
    prev = {k: (None if v is None else v[:, 0].contiguous()) for k, v in inputs.items()
            if k in ("u", "Bm")}
    cur = {k: (None if v is None else (v[:, 1].contiguous() if k in ("u", "delta", "lam", "theta", "Bm", "Cm")
                                        else v)) for k, v in inputs.items()}
    h_shape = (w.batch, w.dim, w.dstate, 2) if w.is_complex else (w.batch, w.dim, w.dstate)
    g = torch.Generator(device=dev).manual_seed(1)
    h = torch.randn(h_shape, generator=g, device=dev)
    h_start = h.clone()
    y = torch.empty_like(cur["u"])
    stream = torch.cuda.current_stream(dev)
    trap = w.disc == "trap"

    def step():
        ssm_scan_step(cur["u"], cur["delta"], cur["A"], cur["Bm"], cur["Cm"], cur["Dskip"], cur["theta"],
                      cur["lam"], h=h, u_prev=prev["u"] if trap else None, B_prev=prev["Bm"] if trap else None,
                      disc=w.disc, y=y, stream=stream.cuda_stream)

    timing = _timed(torch, stream, step, args.steps, args.warmup, "decode steps")
    ms = timing.ms
    alg_bytes = decode_algorithmic_bytes(w)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.batch * w.dim / (ms * 1e-3), "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": 1, "dstate": w.dstate,
                   "disc": w.disc, "complex": w.is_complex, "io_dtype": w.io_dtype, "algo": "step"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w.name, "step"),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a channel sample")
        out["cpu_baseline"] = cpu_baseline_decode(inputs, w, h_start, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_backward(args, w, torch, dev):
    import numpy as np

    from selective_state_space_42_amd.inputs import make_inputs
    from selective_state_space_42_amd.scan import make_desc, ssm_scan_bwd, ssm_scan_bwd_workspace_bytes

    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_inputs(w, device=dev)
    g = torch.Generator(device=dev).manual_seed(2)
    dy = torch.randn(inputs["u"].shape, generator=g, device=dev).to(inputs["u"].dtype)
    desc = make_desc(w.batch, w.seqlen, w.dim, w.dstate, inputs["u"].dtype, w.disc, w.is_complex)
    ws = torch.empty(max(ssm_scan_bwd_workspace_bytes(desc), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ssm_scan_bwd(inputs["u"], inputs["delta"], inputs["A"], inputs["Bm"], inputs["Cm"], inputs["Dskip"],
                            inputs["theta"], inputs["lam"], dy=dy, disc=w.disc, workspace=ws,
                            stream=stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the binding allocates the gradient tensors on every call; the timed loop
    # calls the library directly on one set of them
    grads = step()
    torch.cuda.synchronize()
    import ctypes

    from selective_state_space_42_amd import scan as _scan
    ptr = _scan._ptr
    lib = _scan._lib()

    def call():
        st = lib.ssm_scan_bwd(ctypes.byref(desc), ptr(inputs["u"]), ptr(inputs["delta"]), ptr(inputs["A"]),
                              ptr(inputs["Bm"]), ptr(inputs["Cm"]), ptr(inputs["Dskip"]), ptr(inputs["theta"]),
                              ptr(inputs["lam"]), None, ptr(dy), None,
                              *(ptr(grads[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dtheta", "dlambda")),
                              None, ptr(ws), ws.numel(), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"ssm_scan_bwd status {st}")

    timing = _timed(torch, stream, call, args.steps, 0, "backward passes")
    ms = timing.ms
    alg = backward_algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.batch * w.seqlen * w.dim / (ms * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                   "disc": w.disc, "complex": w.is_complex, "io_dtype": w.io_dtype, "algo": "backward"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w.name, "backward"),
                     "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from selective_state_space_42_amd.inputs import channel_sample

        log("timing the fp64 oracle's backward on a channel sample")
        spent, tc, nch = 0.0, 0, 0
        order = np.random.default_rng(0).permutation(w.dim).tolist()
        dyh = None
        for c in order:
            x = channel_sample(inputs, [c])
            dyh = dy.index_select(2, torch.as_tensor([c], device=dev)).float().cpu().double().numpy()
            t0 = time.perf_counter()
            oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                            disc=w.disc, is_complex=w.is_complex, dy=dyh)
            spent += time.perf_counter() - t0
            tc += w.batch * w.seqlen
            nch += 1
            if spent >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {
            "value": tc / spent, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": f"{nch} of {w.dim} channels (random, seed 0), one at a time, every batch row and step: "
                      f"{tc} tokens*channels in {spent:.1f} s of the single-threaded fp64 C oracle backward"}
    print(json.dumps(out), flush=True)


def bench_ssd(args, w, torch, dev):
    import numpy as np

    from selective_state_space_42_amd.inputs import make_ssd_inputs, ssd_as_scan
    from selective_state_space_42_amd.scan import make_ssd_desc, ssm_ssd_fwd, ssm_ssd_workspace_bytes

    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_ssd_inputs(w, device=dev)
    y = torch.empty_like(inputs["u"])
    h_last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
    desc = make_ssd_desc(w.batch, w.seqlen, w.dim, w.dstate, w.headdim, inputs["u"].dtype)
    ws = torch.empty(max(ssm_ssd_workspace_bytes(desc), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm_ssd_fwd(inputs["u"], inputs["delta"], inputs["A"], inputs["Bm"], inputs["Cm"], inputs["Dskip"],
                    headdim=w.headdim, y=y, h_last=h_last, workspace=ws, stream=stream.cuda_stream)

    timing = _timed(torch, stream, step, args.steps, args.warmup, "SSD passes")
    ms = timing.ms
    alg = ssd_algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.batch * w.seqlen * w.dim / (ms * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                   "headdim": w.headdim, "disc": "euler", "complex": False, "io_dtype": w.io_dtype, "algo": "ssd"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w.name, "ssd"),
                     "algorithmic_bytes_per_launch": alg},
        # the products' side: algorithmic matrix flops over the step time against the bf16 MFMA peak
        "roofline_mfma": {"bound": "mfma", "achieved": ssd_algorithmic_flops(w) / (ms * 1e-3) / 1e12,
                          "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                          "frac": ssd_algorithmic_flops(w) / (ms * 1e-3) / 1e12 / PEAK_BF16_MFMA_TFLOPS,
                          "algorithmic_flops_per_launch": ssd_algorithmic_flops(w)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        log("timing the fp64 oracle on a channel sample")
        threads = max(1, min(os.cpu_count() or 1, 64))
        order = np.random.default_rng(0).permutation(w.dim).tolist()
        spent, tc, used, err, groups = 0.0, 0, 0, 0.0, 0
        for g0 in range(0, w.dim, threads):
            idx = sorted(order[g0:g0 + threads])
            x = ssd_as_scan(inputs, w, idx)
            t0 = time.perf_counter()
            y_ref, _ = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], disc="euler",
                                   is_complex=False, nthreads=len(idx))
            spent += time.perf_counter() - t0
            tc += w.batch * w.seqlen * len(idx)
            used = max(used, len(idx))
            groups += 1
            yg = y.index_select(2, torch.as_tensor(idx, device=dev)).float().cpu().double().numpy()
            err = max(err, float(np.max(np.abs(yg - y_ref)) / np.max(np.abs(y_ref))))
            if spent >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {
            "value": tc / spent, "unit": UNIT, "cores": used, "kind": "oracle",
            "sample": f"{tc // (w.batch * w.seqlen)} of {w.dim} channels (random, seed 0) in {groups} group(s), "
                      f"every batch row and step, as the equivalent scan: {tc} tokens*channels in {spent:.1f} s "
                      f"of fp64 C oracle time on {used} pthreads",
            "parity_err_y_on_sample": err}
    print(json.dumps(out), flush=True)





def bench_mimo(args, w, torch, dev):
    import numpy as np

    from selective_state_space_42_amd.inputs import channel_sample, make_mimo_inputs
    from selective_state_space_42_amd.scan import make_mimo_desc, ssm_mimo_fwd, ssm_mimo_workspace_bytes

    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_mimo_inputs(w, device=dev)
    y = torch.empty_like(inputs["u"])
    h_last = torch.empty((w.batch, w.dim, w.dstate) + ((2,) if w.is_complex else ()), dtype=torch.float32,
                         device=dev)
    desc = make_mimo_desc(w.batch, w.seqlen, w.dim, w.dstate, w.rank, inputs["u"].dtype, w.disc, w.is_complex)
    ws_bytes = ssm_mimo_workspace_bytes(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm_mimo_fwd(inputs["u"], inputs["delta"], inputs["A"], inputs["Bm"], inputs["Cm"], inputs["Dskip"],
                     inputs["theta"], inputs["lam"], disc=w.disc, y=y, h_last=h_last, workspace=ws,
                     stream=stream.cuda_stream)

    timing = _timed(torch, stream, step, args.steps, args.warmup)
    ms = timing.ms
    log(f"timed {args.steps} MIMO scans: {ms:.3f} ms each")
    alg = mimo_algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.batch * w.seqlen * w.dim / (ms * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                   "rank": w.rank, "disc": w.disc, "complex": w.is_complex, "io_dtype": w.io_dtype,
                   "algo": "mimo", "workspace_bytes": ws_bytes},
        # the prefill's vector arithmetic bounds it (fp32 recurrences of rank R
        # per state); the HBM side is kept beside it
        "roofline": {"bound": "alu", "achieved": mimo_algorithmic_flops(w) / (ms * 1e-3) / 1e12,
                     "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                     "frac": mimo_algorithmic_flops(w) / (ms * 1e-3) / 1e12 / PEAK_FP32_VECTOR_TFLOPS,
                     "traffic": None, "algorithmic_flops_per_launch": mimo_algorithmic_flops(w)},
        "roofline_hbm": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w.name, "mimo"),
                         "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        log("timing the fp64 MIMO oracle on a channel sample")
        threads = max(1, min(os.cpu_count() or 1, 64))
        order = np.random.default_rng(0).permutation(w.dim).tolist()
        spent, tc, used, err, groups = 0.0, 0, 0, 0.0, 0
        for g0 in range(0, w.dim, threads):
            idx = sorted(order[g0:g0 + threads])
            x = channel_sample(inputs, idx)
            t0 = time.perf_counter()
            y_ref, _ = oracle.scan_mimo(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"],
                                        x["lam"], disc=w.disc, is_complex=w.is_complex, nthreads=len(idx))
            spent += time.perf_counter() - t0
            tc += w.batch * w.seqlen * len(idx)
            used = max(used, len(idx))
            groups += 1
            yg = y.index_select(2, torch.as_tensor(idx, device=dev)).float().cpu().double().numpy()
            err = max(err, float(np.max(np.abs(yg - y_ref)) / np.max(np.abs(y_ref))))
            if spent >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {
            "value": tc / spent, "unit": UNIT, "cores": used, "kind": "oracle",
            "sample": f"{tc // (w.batch * w.seqlen)} of {w.dim} channels (random, seed 0) in {groups} group(s), "
                      f"every batch row and step, R={w.rank}: {tc} tokens*channels in {spent:.1f} s of fp64 C "
                      f"oracle time on {used} pthreads",
            "parity_err_y_on_sample": err}
    print(json.dumps(out), flush=True)


def bench_mimo_decode(args, w, torch, dev):
    import numpy as np

    from selective_state_space_42_amd.inputs import channel_sample, make_mimo_inputs
    from selective_state_space_42_amd.scan import ssm_mimo_step

    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_mimo_inputs(w, device=dev)
    per_step = ("u", "delta", "lam", "theta", "Bm", "Cm")
    prev = {k: inputs[k][:, 0].contiguous() for k in ("u", "Bm")}
    cur = {k: (v[:, 1].contiguous() if k in per_step and v is not None else v) for k, v in inputs.items()}
    g = torch.Generator(device=dev).manual_seed(1)
    h = torch.randn((w.batch, w.dim, w.dstate) + ((2,) if w.is_complex else ()), generator=g, device=dev)
    h_start = h.clone()
    y = torch.empty_like(cur["u"])
    stream = torch.cuda.current_stream(dev)
    trap = w.disc == "trap"

    def step():
        ssm_mimo_step(cur["u"], cur["delta"], cur["A"], cur["Bm"], cur["Cm"], cur["Dskip"], cur["theta"],
                      cur["lam"], h=h, u_prev=prev["u"] if trap else None, B_prev=prev["Bm"] if trap else None,
                      disc=w.disc, y=y, stream=stream.cuda_stream)

    timing = _timed(torch, stream, step, args.steps, args.warmup)
    ms = timing.ms
    log(f"timed {args.steps} MIMO decode steps: {ms * 1e3:.2f} us/step")
    alg = mimo_decode_algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": w.batch * w.dim / (ms * 1e-3), "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": 1, "dstate": w.dstate,
                   "rank": w.rank, "disc": w.disc, "complex": w.is_complex, "io_dtype": w.io_dtype,
                   "algo": "mimo_step"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w.name, "mimo_step"),
                     "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        log("timing the fp64 MIMO oracle on one decode step of a channel sample")
        threads = max(1, min(os.cpu_count() or 1, 64))
        idx = sorted(np.random.default_rng(0).permutation(w.dim)[:max(threads, 64)].tolist())
        x = channel_sample(inputs, idx)
        first = {k: (v[:, 0:1] if k in per_step and v is not None else v) for k, v in x.items()}
        second = {k: (v[:, 1:2] if k in per_step and v is not None else v) for k, v in x.items()}
        q0 = None
        if trap:  # q of the previous step, the oracle's own sum over the ranks
            _, _, q0 = oracle.scan_mimo(*(first[k] for k in ("u", "delta", "A", "Bm", "Cm", "Dskip", "theta",
                                                              "lam")), disc=w.disc, is_complex=w.is_complex,
                                        return_q=True)
        h0 = h_start[:, idx].float().cpu().double().numpy()
        spent, calls = 0.0, 0
        while spent < args.cpu_seconds:
            t0 = time.perf_counter()
            oracle.scan_mimo(*(second[k] for k in ("u", "delta", "A", "Bm", "Cm", "Dskip", "theta", "lam")),
                             disc=w.disc, is_complex=w.is_complex, h0=h0, q0=q0, nthreads=threads)
            spent += time.perf_counter() - t0
            calls += 1
        tc = calls * w.batch * len(idx)
        out["cpu_baseline"] = {
            "value": tc / spent, "unit": UNIT, "cores": min(threads, len(idx)), "kind": "oracle",
            "sample": f"{len(idx)} of {w.dim} channels (random, seed 0), every batch row, one MIMO decode step "
                      f"(R={w.rank}) from a given state, repeated {calls} times: {tc} tokens*channels in "
                      f"{spent:.1f} s of fp64 C oracle time"}
    print(json.dumps(out), flush=True)


def copy_calibration(torch, dev, nbytes: int, steps: int, warmup: int):
    """A plain copy of known size: reads and writes `nbytes` per launch."""
    n = (nbytes + 15) // 16 * 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": steps + warmup,
                      "ms_per_copy": ms, "GBps": 8 * n / (ms * 1e-3) / 1e9}), flush=True)


def stream_calibration(torch, dev, steps: int, warmup: int):
    """The practical HBM ceiling for the scan's traffic shape, measured by the
    library's own read-dominant stream kernel (ssm_calibrate_stream): 19 bytes
    read per byte written (95 % reads, like the scan), 45.9 GB read and
    2.4 GB written per launch, far beyond the L2s and the 256 MB MALL.  Both
    the default and the non-temporal cache policy are timed; the kernel also
    reports the sustained shader clock (s_memtime against the 100 MHz
    s_memrealtime counter)."""
    from selective_state_space_42_amd.scan import ssm_calibrate_stream

    ratio, dst_bytes = 19, 9 << 28
    src = torch.empty(ratio * dst_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty(dst_bytes // 4, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    moved = (ratio + 1) * dst_bytes
    out = {"calibration": "hbm_read_stream", "read_bytes": ratio * dst_bytes, "write_bytes": dst_bytes,
           "reads_per_write": ratio, "peak_GBps": PEAK_HBM_GBS}
    for name, nt in (("default", False), ("nontemporal", True)):
        t = _timed(torch, stream, lambda: ssm_calibrate_stream(src, dst, nontemporal=nt, clocks=clocks,
                                                               stream=stream.cuda_stream),
                   steps, warmup, f"{name} stream launches")
        ticks = clocks.cpu().tolist()
        out[name] = {"GBps_median": moved / (t.median * 1e-3) / 1e9, "GBps_best": moved / (t.min * 1e-3) / 1e9,
                     "frac_of_peak_median": moved / (t.median * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "timing": t.record(),
                     "sustained_clock_MHz": ticks[0] / ticks[1] * 100.0 if ticks[1] > 0 else None}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--algo", default="auto", choices=["auto", "sequential", "chunked", "sweep"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (ssm_scan_bwd) instead")
    ap.add_argument("--stream-calibration", action="store_true",
                    help="instead of the scan, time the library's read-dominant HBM stream kernel (95 %% reads, "
                         "48 GB per launch): the practical bandwidth ceiling the scan is compared with")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the scan, time a plain device-to-device copy of BYTES bytes "
                         "(the known-size kernel that HBM byte counters are scaled against)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (use --gpus 1): the scan shards along batch rows and channels "
              "with no communication between GPUs, so N GPUs each run this one-GPU measurement on their share.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_42_amd.inputs import (DECODE_WORKLOADS, MIMO_DECODE_WORKLOADS, MIMO_WORKLOADS,
                                                     SSD_WORKLOADS, WORKLOADS, make_inputs)
    from selective_state_space_42_amd.scan import make_desc, ssm_scan_algo, ssm_scan_fwd, ssm_scan_workspace_bytes

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration, args.steps, args.warmup)
        return
    if args.stream_calibration:
        stream_calibration(torch, dev, args.steps, args.warmup)
        return
    if args.workload in DECODE_WORKLOADS:
        bench_decode(args, DECODE_WORKLOADS[args.workload], torch, dev)
        return
    if args.workload in SSD_WORKLOADS:
        bench_ssd(args, SSD_WORKLOADS[args.workload], torch, dev)
        return
    if args.workload in MIMO_WORKLOADS:
        bench_mimo(args, MIMO_WORKLOADS[args.workload], torch, dev)
        return
    if args.workload in MIMO_DECODE_WORKLOADS:
        bench_mimo_decode(args, MIMO_DECODE_WORKLOADS[args.workload], torch, dev)
        return
    w = WORKLOADS[args.workload]
    if args.backward:
        bench_backward(args, w, torch, dev)
        return
    log(f"generating {w.name} on {torch.cuda.get_device_name(dev)}")
    inputs = make_inputs(w, device=dev)
    torch.cuda.synchronize()
    y = torch.empty_like(inputs["u"])
    h_shape = (w.batch, w.dim, w.dstate, 2) if w.is_complex else (w.batch, w.dim, w.dstate)
    h_last = torch.empty(h_shape, dtype=torch.float32, device=dev)
    desc = make_desc(w.batch, w.seqlen, w.dim, w.dstate, inputs["u"].dtype, w.disc, w.is_complex, args.algo)
    ws_bytes = ssm_scan_workspace_bytes(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm_scan_fwd(inputs["u"], inputs["delta"], inputs["A"], inputs["Bm"], inputs["Cm"], inputs["Dskip"],
                     inputs["theta"], inputs["lam"], disc=w.disc, y=y, h_last=h_last,
                     workspace=ws if ws_bytes else None, algo=args.algo, stream=stream.cuda_stream)

    timing = _timed(torch, stream, step, args.steps, args.warmup)
    ms = timing.ms

    tc = w.batch * w.seqlen * w.dim
    alg_bytes = algorithmic_bytes(w)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    algo_used = ssm_scan_algo(desc)
    traffic = traffic_from_profile(w.name, algo_used)

    out = {
        "metric": METRIC, "value": tc / (ms * 1e-3), "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "timing": timing.record(), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                   "disc": w.disc, "complex": w.is_complex, "io_dtype": w.io_dtype, "algo": algo_used},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a channel sample")
        out["cpu_baseline"] = cpu_baseline(inputs, w, y, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
