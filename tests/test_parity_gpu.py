"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small and ragged shapes are compared element by element on every output;
the full-size workloads are run in the launch configuration bench.py times
(algo "auto") and compared on a deterministic sample of channels (every batch
row, every step, every state of those channels), which the oracle computes
one channel at a time.
"""
import glob
import os

import numpy as np
import pytest
import torch

from parity_util import TOL, check_workload, rel_err, rel_err_complex, run_gpu
from selective_state_space_42_amd.inputs import WORKLOADS, make_inputs
from selective_state_space_42_amd.scan import ScanError

pytestmark = pytest.mark.gpu

REAL_F32 = WORKLOADS["real_zoh_b8_d1536_l2048_n16"]
CPLX_F32 = WORKLOADS["complex_euler_b8_d2048_l4096_n16"]
CPLX_BF16 = WORKLOADS["complex_trap_bf16_b4_d2560_l8192_n16"]

# every supported (disc, complex) pair in both I/O dtypes
MODES = {
    "real_zoh_f32": REAL_F32,
    "real_zoh_bf16": REAL_F32.scaled(io_dtype="bf16"),
    "real_euler_f32": REAL_F32.scaled(disc="euler"),
    "real_trap_bf16": REAL_F32.scaled(disc="trap", io_dtype="bf16"),
    "real_trap_f32": REAL_F32.scaled(disc="trap"),
    "complex_euler_f32": CPLX_F32,
    "complex_euler_bf16": CPLX_F32.scaled(io_dtype="bf16"),
    "complex_trap_bf16": CPLX_BF16,
    "complex_trap_f32": CPLX_BF16.scaled(io_dtype="f32"),
}
ALGOS = ["sequential", "chunked", "sweep"]


def _run(w, algo, **kw):
    try:
        err_y, err_h, tol = check_workload(w, seed=123, algo=algo, **kw)
    except ScanError as e:
        if e.status == 2 and algo in ("chunked", "sweep"):
            pytest.skip(f"{algo} kernel does not support this case: {e}")
        raise
    print(f"{w.name} algo={algo} err_y={err_y:.3e} err_h={err_h:.3e} tol={tol:g}", flush=True)
    assert err_y <= tol and err_h <= tol, (err_y, err_h, tol)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", list(MODES))
def test_small_ragged(mode, algo):
    """B=2, D=37, L=333 (not a multiple of any tile), N=16: several tiles and a ragged tail."""
    w = MODES[mode].scaled(name=f"{mode}_b2_d37_l333", batch=2, dim=37, seqlen=333)
    _run(w, algo)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 1, 4, 16), (3, 5, 1, 16), (1, 65, 129, 16), (2, 7, 64, 4),
                                   (1, 130, 3, 3), (2, 257, 5, 1), (1, 64, 16, 8)])
@pytest.mark.parametrize("mode", ["real_zoh_f32", "complex_euler_f32", "complex_trap_bf16"])
def test_edge_shapes(mode, shape, algo):
    """(B, L, D, N) edge cases: L = 1, D = 1, N = 1, ragged channel groups, N < 16."""
    B, L, D, N = shape
    w = MODES[mode].scaled(name=f"{mode}_b{B}_l{L}_d{D}_n{N}", batch=B, seqlen=L, dim=D, dstate=N)
    _run(w, algo)


@pytest.mark.parametrize("N", [17, 33, 64])
def test_large_dstate_sequential(N):
    w = MODES["complex_trap_bf16"].scaled(name=f"n{N}", batch=1, dim=6, seqlen=97, dstate=N)
    _run(w, "sequential")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("drop", [("theta",), ("Dskip",), ("h_last",)])
def test_optional_arguments(drop, algo):
    """theta = NULL (theta = 0), D = NULL (no skip term), h_last = NULL (not written)."""
    w = MODES["complex_trap_f32"].scaled(name="optional", batch=2, dim=9, seqlen=150)
    _run(w, algo, drop=drop)


@pytest.mark.parametrize("algo", ALGOS)
def test_long_sequence_many_tiles(algo):
    """A long sequence with few channels: thousands of tiles along L."""
    w = MODES["complex_trap_bf16"].scaled(name="long", batch=1, dim=16, seqlen=1 << 16)
    _run(w, algo, d_index=list(range(16)))


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("scale", [0.5, 8.0, 3000.0])
@pytest.mark.parametrize("mode", ["complex_euler_f32", "complex_trap_bf16"])
def test_wide_rotation_angles(mode, scale, algo):
    """theta = scale * U(-pi, pi): angles past pi/4 (the fp32 path's reduced
    range) and past many revolutions."""
    w = MODES[mode].scaled(name=f"{mode}_theta{scale:g}", batch=2, dim=19, seqlen=300, theta_scale=scale)
    _run(w, algo)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", ["real_zoh_f32", "real_trap_f32", "complex_euler_f32", "complex_trap_bf16"])
def test_degenerate_values(mode, algo):
    """Degenerate values the method admits, mixed into ordinary inputs: A = 0
    for some states (no decay; ZOH's weight becomes delta), delta = 0 at some
    steps (the state is held and nothing enters), lambda exactly 0 and 1 (the
    trapezoid's two one-sided rules) and theta = 0 for some states."""
    w = MODES[mode].scaled(name=f"{mode}_degenerate", batch=2, dim=21, seqlen=257)
    inp = make_inputs(w, 31, device="cuda")
    A = inp["A"].clone()
    A[::3, 1::4] = 0.0
    delta = inp["delta"].clone()
    delta[:, 5::17] = 0
    inputs = dict(inp, A=A, delta=delta)
    if inp["lam"] is not None:
        lam = inp["lam"].clone()
        lam[:, ::11] = 0
        lam[:, 3::11] = 1
        inputs["lam"] = lam
    if inp["theta"] is not None:
        theta = inp["theta"].clone()
        theta[..., ::5] = 0
        inputs["theta"] = theta
    _run(w, algo, inputs=inputs)


GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.npz")))


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden_fixtures(path, algo):
    z = np.load(path)
    disc, cplx, io = (str(v) for v in z["meta"])
    dt = torch.float32 if io == "f32" else torch.bfloat16

    def dev(k, dtype):
        return None if k not in z.files else torch.tensor(z[k], dtype=dtype, device="cuda")
    inputs = dict(u=dev("u", dt), delta=dev("delta", dt), A=dev("A", torch.float32), Bm=dev("Bm", dt),
                  Cm=dev("Cm", dt), Dskip=dev("Dskip", torch.float32), theta=dev("theta", dt), lam=dev("lam", dt))
    try:
        y, h = run_gpu(inputs, disc, algo)
    except ScanError as e:
        if e.status == 2 and algo in ("chunked", "sweep"):
            pytest.skip(str(e))
        raise
    ey = rel_err(y.float().cpu().double().numpy(), z["y"])
    eh = rel_err_complex(h.cpu().double().numpy(), z["h_last"]) if cplx == "1" else rel_err(
        h.cpu().double().numpy(), z["h_last"])
    print(f"{os.path.basename(path)} {algo} err_y={ey:.3e} err_h={eh:.3e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]


def _sample(D, k):
    return sorted(set(np.linspace(0, D - 1, k).astype(int).tolist()))


@pytest.mark.parametrize("name,k", [
    ("real_zoh_b1_d4_l64_n4", 4),
    ("real_zoh_b8_d1536_l2048_n16", 24),
    ("complex_euler_b8_d2048_l4096_n16", 16),
    ("complex_trap_bf16_b4_d2560_l8192_n16", 16),
    ("complex_trap_bf16_b1_d1024_l1048576_n16", 8),
])
def test_full_size_workloads(name, k):
    """The five workloads at full size, algo auto (as bench.py runs them)."""
    w = WORKLOADS[name]
    try:
        _run(w, "auto", d_index=_sample(w.dim, k))
    finally:
        torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["complex_euler_f32", "complex_trap_bf16"])
def test_sweep_unaligned_bc(mode):
    """Complex B and C that start one element past a whole (re, im) entry: the
    lane sweep then loads each part separately."""
    w = MODES[mode].scaled(name=f"{mode}_unaligned", batch=2, dim=13, seqlen=200)
    inp = make_inputs(w, 17, device="cuda")

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % (2 * t.element_size()) != 0
        return v
    _run(w, "sweep", inputs=dict(inp, Bm=shifted(inp["Bm"]), Cm=shifted(inp["Cm"])))


@pytest.mark.parametrize("mode", ["complex_euler_f32", "complex_euler_bf16", "complex_trap_bf16"])
@pytest.mark.parametrize("batch,dim", [(2, 4096), (4, 4093)])
def test_sweep_wide_workgroups(mode, batch, dim):
    """2048 and 4096 waves of 4 channels (the second with a ragged last
    group): on a 256-CU GPU the complex sweep packs 8 and 16 waves per
    workgroup, which then meet at a barrier every block."""
    w = MODES[mode].scaled(name=f"{mode}_b{batch}_d{dim}_wide", batch=batch, dim=dim, seqlen=37)
    _run(w, "sweep")
