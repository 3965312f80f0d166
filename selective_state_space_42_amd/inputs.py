"""Seeded synthetic inputs for the selective scan.

This module only draws random tensors with the shapes and distributions of the
scan's workloads; it contains none of the scan's arithmetic.  Both the HIP
path (tests, bench) and the fp64 oracle consume what it produces: the oracle
always reads the *stored* values (after rounding to the I/O dtype), so parity
never depends on the random stream itself.

Workloads (row-major layouts; complex values interleaved re,im):
  u, delta, lambda : (B, L, D)      io dtype
  A                : (D, N)         fp32
  Bm, Cm           : (B, L, N) real, or (B, L, N, 2) complex   io dtype
  Dskip            : (D,)           fp32
  theta            : (B, L, D, N)   io dtype (complex workloads only)

Draw order (fixed): u, delta pre-activation, A (when random), B re, B im,
C re, C im, Dskip, theta, lambda pre-activation.  Values are drawn in fp32 and
rounded to nearest-even into the I/O dtype; A and Dskip stay fp32.  Large
tensors are filled in fixed-size chunks of their flat storage so that the
transient memory stays bounded and the realisation does not depend on it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_CHUNK = 1 << 26  # elements per generator call


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int          # D, channels
    seqlen: int       # L
    dstate: int       # N
    disc: str         # "zoh" | "euler" | "trap"
    is_complex: bool
    io_dtype: str     # "f32" | "bf16"
    delta_mu: float   # delta = softplus(N(delta_mu, delta_sigma))
    delta_sigma: float
    a_kind: str       # "neg_index": A[d,n] = -(n+1);  "neg_exp_uniform": A = -exp(U(-3,0))
    bc_var: float     # variance of B, C (real) or of each of re/im (complex)
    theta_scale: float = 0.1  # theta = theta_scale * U(-pi, pi)
    rank: int = 0     # MIMO workloads: R inputs and outputs per token and channel (0: single-input layout)

    @property
    def shape(self):
        return (self.batch, self.seqlen, self.dim, self.dstate)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Where the complex workloads leave delta, u and Dskip
# unstated they take the Mamba-1-style workload's distributions; "re/im ~
# N(0, 1/2)" is read as variance 1/2 for each part.
WORKLOADS = {
    "real_zoh_b1_d4_l64_n4": Workload(
        "real_zoh_b1_d4_l64_n4", 1, 4, 64, 4, "zoh", False, "f32", -2.0, 0.5, "neg_index", 1.0),
    "real_zoh_b8_d1536_l2048_n16": Workload(
        "real_zoh_b8_d1536_l2048_n16", 8, 1536, 2048, 16, "zoh", False, "f32", -3.0, 0.5, "neg_index", 1.0),
    "complex_euler_b8_d2048_l4096_n16": Workload(
        "complex_euler_b8_d2048_l4096_n16", 8, 2048, 4096, 16, "euler", True, "f32", -3.0, 0.5,
        "neg_exp_uniform", 0.5),
    "complex_trap_bf16_b4_d2560_l8192_n16": Workload(
        "complex_trap_bf16_b4_d2560_l8192_n16", 4, 2560, 8192, 16, "trap", True, "bf16", -3.0, 0.5,
        "neg_exp_uniform", 0.5),
    "complex_trap_bf16_b1_d1024_l1048576_n16": Workload(
        "complex_trap_bf16_b1_d1024_l1048576_n16", 1, 1024, 1 << 20, 16, "trap", True, "bf16", -4.0, 0.5,
        "neg_exp_uniform", 0.5),
}
WORKLOAD_ORDER = list(WORKLOADS)

# Decode-step workloads: one token per call with the state kept in memory, a
# serving batch of B sequences.  seqlen = 2 holds the previous step (whose u
# and B the trapezoid needs) and the current one; the fields are drawn as for
# the complex exp-trapezoidal bf16 workload.
DECODE_WORKLOADS = {
    "decode_complex_trap_bf16_b256_d2560_n16": Workload(
        "decode_complex_trap_bf16_b256_d2560_n16", 256, 2560, 2, 16, "trap", True, "bf16", -3.0, 0.5,
        "neg_exp_uniform", 0.5),
}
SEED_BASE = 42


def seed_of(name: str) -> int:
    return SEED_BASE + WORKLOAD_ORDER.index(name) if name in WORKLOADS else SEED_BASE


def torch_dtype(io_dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[io_dtype]


def _fill(out: torch.Tensor, gen: torch.Generator, kind: str, a: float = 0.0, b: float = 1.0,
          post=None):
    """Fill `out` (contiguous) chunk by chunk with fp32 draws, then round to its dtype.

    kind "normal": N(a, b) (b = std); kind "uniform": U(a, b).
    `post` is an optional elementwise map applied in fp32 before rounding.
    """
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - s)
        if kind == "normal":
            v = torch.randn(n, generator=gen, device=out.device, dtype=torch.float32)
            v = v * b + a
        else:
            v = torch.rand(n, generator=gen, device=out.device, dtype=torch.float32)
            v = v * (b - a) + a
        if post is not None:
            v = post(v)
        flat[s:s + n] = v.to(out.dtype)
    return out


def make_inputs(w: Workload, seed: Optional[int] = None, device="cpu") -> dict:
    """Draw one seeded instance of workload `w` on `device`."""
    if seed is None:
        seed = seed_of(w.name)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    io = torch_dtype(w.io_dtype)
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    kw = dict(device=device)

    u = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", 0.0, 1.0)
    delta = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", w.delta_mu, w.delta_sigma,
                  post=torch.nn.functional.softplus)
    if w.a_kind == "neg_index":
        A = -(torch.arange(1, N + 1, dtype=torch.float32, device=device)).repeat(D, 1).contiguous()
    else:
        A = _fill(torch.empty((D, N), dtype=torch.float32, **kw), gen, "uniform", -3.0, 0.0,
                  post=lambda v: -torch.exp(v))
    std = math.sqrt(w.bc_var)
    if w.is_complex:
        Bre = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
        Bim = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
        Cre = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
        Cim = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
        Bm = torch.stack([Bre, Bim], dim=-1).contiguous()
        Cm = torch.stack([Cre, Cim], dim=-1).contiguous()
        del Bre, Bim, Cre, Cim
    else:
        Bm = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
        Cm = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, std)
    Dskip = _fill(torch.empty((D,), dtype=torch.float32, **kw), gen, "normal", 0.0, 1.0)
    theta = None
    if w.is_complex:
        theta = _fill(torch.empty((B, L, D, N), dtype=io, **kw), gen, "uniform",
                      -math.pi * w.theta_scale, math.pi * w.theta_scale)
    lam = None
    if w.disc == "trap":
        lam = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", 0.0, 1.0, post=torch.sigmoid)
    return dict(u=u, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, theta=theta, lam=lam)


def channel_sample(inputs: dict, d_index) -> dict:
    """Copy the inputs of a subset of channels to host fp64 numpy arrays.

    The subset keeps every batch row and every step; B and C (shared by all
    channels) are copied whole.  Widening fp32/bf16 to fp64 is exact.
    """
    idx = torch.as_tensor(d_index, dtype=torch.long, device=inputs["u"].device)

    def host(t):
        return None if t is None else t.float().cpu().double().numpy()

    out = dict(
        u=host(inputs["u"].index_select(2, idx)),
        delta=host(inputs["delta"].index_select(2, idx)),
        A=host(inputs["A"].index_select(0, idx)),
        Bm=host(inputs["Bm"]),
        Cm=host(inputs["Cm"]),
        Dskip=None if inputs["Dskip"] is None else host(inputs["Dskip"].index_select(0, idx)),
        theta=None if inputs["theta"] is None else host(inputs["theta"].index_select(2, idx)),
        lam=None if inputs["lam"] is None else host(inputs["lam"].index_select(2, idx)),
    )
    return out


def all_channels(inputs: dict) -> dict:
    """Host fp64 copies of every input (small workloads only)."""
    return channel_sample(inputs, range(inputs["u"].shape[2]))


# ---- the state-space dual (SSD) setting: heads of `headdim` channels sharing
# a step size per (b, t, head) and a scalar A per head; real state,
# exponential-Euler b-terms, B and C shared by all heads, bf16 I/O.  Fields are
# drawn like the other workloads': u, B, C, D ~ N(0, 1), delta per head =
# softplus(N(-3, 0.5)), A per head = -exp(U(-3, 0)).
@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    headdim: int = 64
    io_dtype: str = "bf16"
    delta_mu: float = -3.0
    delta_sigma: float = 0.5

    @property
    def heads(self):
        return self.dim // self.headdim

    def scaled(self, **kw) -> "SsdWorkload":
        return dataclasses.replace(self, **kw)


SSD_WORKLOADS = {
    "ssd_real_bf16_b4_d2560_l8192_n16_p64": SsdWorkload("ssd_real_bf16_b4_d2560_l8192_n16_p64", 4, 2560, 8192, 16),
}


def make_ssd_inputs(w: SsdWorkload, seed: Optional[int] = None, device="cpu") -> dict:
    """One seeded instance of an SSD workload: u (B,L,D), delta (B,L,H),
    A (H,), Bm, Cm (B,L,N), Dskip (D,)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_BASE + 100 if seed is None else seed)
    io = torch_dtype(w.io_dtype)
    B, L, D, N, H = w.batch, w.seqlen, w.dim, w.dstate, w.heads
    kw = dict(device=device)
    u = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", 0.0, 1.0)
    delta = _fill(torch.empty((B, L, H), dtype=io, **kw), gen, "normal", w.delta_mu, w.delta_sigma,
                  post=torch.nn.functional.softplus)
    A = _fill(torch.empty((H,), dtype=torch.float32, **kw), gen, "uniform", -3.0, 0.0, post=lambda v: -torch.exp(v))
    Bm = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, 1.0)
    Cm = _fill(torch.empty((B, L, N), dtype=io, **kw), gen, "normal", 0.0, 1.0)
    Dskip = _fill(torch.empty((D,), dtype=torch.float32, **kw), gen, "normal", 0.0, 1.0)
    return dict(u=u, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip)


def ssd_as_scan(inputs: dict, w: SsdWorkload, d_index=None) -> dict:
    """The same problem in the scan's layout (delta per channel, A per (d, n)),
    for channels d_index (all when None), as host fp64 arrays (exact widening)."""
    D = w.dim
    idx = list(range(D)) if d_index is None else list(d_index)
    heads = torch.as_tensor([d // w.headdim for d in idx], device=inputs["u"].device)
    sel = torch.as_tensor(idx, device=inputs["u"].device)

    def host(t):
        return t.float().cpu().double().numpy()

    return dict(
        u=host(inputs["u"].index_select(2, sel)),
        delta=host(inputs["delta"].index_select(2, heads)),
        A=host(inputs["A"].index_select(0, heads)[:, None].expand(len(idx), w.dstate)),
        Bm=host(inputs["Bm"]), Cm=host(inputs["Cm"]),
        Dskip=host(inputs["Dskip"].index_select(0, sel)), theta=None, lam=None)


# ---- the multi-input multi-output (MIMO) setting: R inputs and outputs per
# token and channel sharing one state; u, y (B, L, D, R) and B, C (B, L, N, R)
# or (B, L, N, R, 2).  R = 4 is the rank the Mamba-3 story's inference table
# quotes.  Fields are drawn as for the complex exp-trapezoidal bf16 workload,
# in the same order, each with its R axis.
MIMO_WORKLOADS = {
    "mimo_complex_trap_bf16_b4_d2560_l8192_n16_r4": Workload(
        "mimo_complex_trap_bf16_b4_d2560_l8192_n16_r4", 4, 2560, 8192, 16, "trap", True, "bf16", -3.0, 0.5,
        "neg_exp_uniform", 0.5, rank=4),
}
# decode steps: seqlen = 2 holds the previous step and the current one
MIMO_DECODE_WORKLOADS = {
    "mimo_decode_complex_trap_bf16_b256_d2560_n16_r4": Workload(
        "mimo_decode_complex_trap_bf16_b256_d2560_n16_r4", 256, 2560, 2, 16, "trap", True, "bf16", -3.0, 0.5,
        "neg_exp_uniform", 0.5, rank=4),
}


def make_mimo_inputs(w: Workload, seed: Optional[int] = None, device="cpu") -> dict:
    """One seeded instance of a MIMO workload: u (B,L,D,R), delta, lam (B,L,D),
    A (D,N), Bm, Cm (B,L,N,R[,2]), Dskip (D,), theta (B,L,D,N)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_BASE + 200 if seed is None else seed)
    io = torch_dtype(w.io_dtype)
    B, L, D, N, R = w.batch, w.seqlen, w.dim, w.dstate, w.rank
    kw = dict(device=device)
    u = _fill(torch.empty((B, L, D, R), dtype=io, **kw), gen, "normal", 0.0, 1.0)
    delta = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", w.delta_mu, w.delta_sigma,
                  post=torch.nn.functional.softplus)
    if w.a_kind == "neg_index":
        A = -(torch.arange(1, N + 1, dtype=torch.float32, device=device)).repeat(D, 1).contiguous()
    else:
        A = _fill(torch.empty((D, N), dtype=torch.float32, **kw), gen, "uniform", -3.0, 0.0,
                  post=lambda v: -torch.exp(v))
    std = math.sqrt(w.bc_var)
    parts = []
    for _ in range(4 if w.is_complex else 2):  # B re, (B im,) C re, (C im)
        parts.append(_fill(torch.empty((B, L, N, R), dtype=io, **kw), gen, "normal", 0.0, std))
    if w.is_complex:
        Bm = torch.stack(parts[:2], dim=-1).contiguous()
        Cm = torch.stack(parts[2:], dim=-1).contiguous()
    else:
        Bm, Cm = parts
    del parts
    Dskip = _fill(torch.empty((D,), dtype=torch.float32, **kw), gen, "normal", 0.0, 1.0)
    theta = None
    if w.is_complex:
        theta = _fill(torch.empty((B, L, D, N), dtype=io, **kw), gen, "uniform",
                      -math.pi * w.theta_scale, math.pi * w.theta_scale)
    lam = None
    if w.disc == "trap":
        lam = _fill(torch.empty((B, L, D), dtype=io, **kw), gen, "normal", 0.0, 1.0, post=torch.sigmoid)
    return dict(u=u, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, theta=theta, lam=lam)
