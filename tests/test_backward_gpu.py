"""GPU parity of the backward pass (ssm_scan_bwd) against the fp64 oracle's
gradients (oracle.scan_bwd, pinned to finite differences in
test_oracle_bwd_pins.py).

Every gradient tensor is compared element by element with
    err = max |g_gpu - g_ref| / max |g_ref|.
The source specifies tolerances for the forward outputs only.  The
gradients are fp32 outputs of fp32 arithmetic on the same (exactly widened)
inputs, so fp32 I/O keeps the forward's 1e-5 (measured: at most 1.6e-6, the
largest on dtheta and dA, whose sums over B*L terms are taken with atomic
adds).  bf16 I/O uses the hardware sin/cos, whose small bias compounds along
the sequence as in the forward scan (measured: at most 7.4e-6); its bar is
1e-4, tighter than the forward's 2e-2 because no output is rounded to bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import rel_err
from selective_state_space_42_amd.inputs import WORKLOADS, all_channels, make_inputs
from selective_state_space_42_amd.scan import ssm_scan_bwd

pytestmark = pytest.mark.gpu

GRAD_TOL = {"f32": 1e-5, "bf16": 1e-4}
_R = WORKLOADS["real_zoh_b8_d1536_l2048_n16"]
_C = WORKLOADS["complex_euler_b8_d2048_l4096_n16"]
MODES = {
    "real_zoh_f32": _R,
    "real_zoh_bf16": _R.scaled(io_dtype="bf16"),
    "real_euler_f32": _R.scaled(disc="euler"),
    "real_trap_f32": _R.scaled(disc="trap"),
    "real_trap_bf16": _R.scaled(disc="trap", io_dtype="bf16"),
    "complex_euler_f32": _C,
    "complex_euler_bf16": _C.scaled(io_dtype="bf16"),
    "complex_trap_f32": _C.scaled(disc="trap"),
    "complex_trap_bf16": _C.scaled(disc="trap", io_dtype="bf16"),
}


def _host(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def _compare(w, inp, dy, dh_last=None, h0=None, label=""):
    g = ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["theta"], inp["lam"],
                     h0, dy=dy, dh_last=dh_last, disc=w.disc, want_dh0=True)
    torch.cuda.synchronize()
    x = all_channels(inp)
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                          disc=w.disc, is_complex=w.is_complex, dy=_host(dy), dh_last=_host(dh_last), h0=_host(h0))
    errs = {}
    for k, r in ref.items():
        if r is None:
            assert g[k] is None or k == "dD", k
            continue
        errs[k] = rel_err(_host(g[k]), r)
    tol = GRAD_TOL[w.io_dtype]
    print(f"{label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) <= tol, (errs, tol)


@pytest.mark.parametrize("mode", list(MODES))
def test_backward_small_ragged(mode):
    """B=2, D=37, L=333 (forty-one 8-step segments and a ragged one, in two
    time chunks of the reverse sweep, the second ragged), N=16."""
    w = MODES[mode].scaled(batch=2, dim=37, seqlen=333)
    inp = make_inputs(w, seed=21, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(3)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    _compare(w, inp, dy, label=mode)


@pytest.mark.parametrize("mode", ["real_trap_f32", "complex_trap_f32", "complex_trap_bf16", "complex_euler_f32"])
def test_backward_with_state_gradients(mode):
    """Nonzero h0 and dh_last; odd N; D not a multiple of the wave's channels."""
    w = MODES[mode].scaled(batch=3, dim=13, seqlen=70, dstate=5)
    inp = make_inputs(w, seed=22, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(4)
    shape = (w.batch, w.dim, w.dstate) + ((2,) if w.is_complex else ())
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    dh = torch.randn(shape, generator=gen, device="cuda")
    h0 = torch.randn(shape, generator=gen, device="cuda")
    _compare(w, inp, dy, dh_last=dh, h0=h0, label=mode)


@pytest.mark.parametrize("mode", ["real_zoh_f32", "real_trap_f32", "complex_trap_f32", "complex_trap_bf16"])
def test_backward_time_chunks(mode):
    """A narrow, long problem: the reverse sweep runs in four time chunks of 256
    steps (the last ragged) chained by the adjoint carry, with nonzero h0 and
    dh_last and odd N."""
    w = MODES[mode].scaled(batch=1, dim=5, seqlen=1000, dstate=7)
    inp = make_inputs(w, seed=25, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    shape = (w.batch, w.dim, w.dstate) + ((2,) if w.is_complex else ())
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    dh = torch.randn(shape, generator=gen, device="cuda")
    h0 = torch.randn(shape, generator=gen, device="cuda")
    _compare(w, inp, dy, dh_last=dh, h0=h0, label=f"chunks {mode}")


@pytest.mark.parametrize("mode", ["real_zoh_f32", "real_trap_bf16", "complex_trap_f32", "complex_trap_bf16"])
def test_backward_workgroup_sums(mode):
    """D a multiple of 16: each workgroup's four waves share the batch row and
    time chunk, and dB, dC are summed over its channels in LDS per segment
    (compared in full here).  Ragged segments, two time chunks, N = 16."""
    w = MODES[mode].scaled(batch=2, dim=32, seqlen=333)
    inp = make_inputs(w, seed=26, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(8)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    _compare(w, inp, dy, label=f"wg sums {mode}")


@pytest.mark.parametrize("mode", ["real_trap_f32", "complex_trap_bf16"])
def test_backward_workgroup_sums_time_chunks_odd_n(mode):
    """The LDS sums with four time chunks, N = 7 (lanes past N add zeros),
    nonzero h0 and dh_last."""
    w = MODES[mode].scaled(batch=1, dim=16, seqlen=1000, dstate=7)
    inp = make_inputs(w, seed=27, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(9)
    shape = (w.batch, w.dim, w.dstate) + ((2,) if w.is_complex else ())
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    dh = torch.randn(shape, generator=gen, device="cuda")
    h0 = torch.randn(shape, generator=gen, device="cuda")
    _compare(w, inp, dy, dh_last=dh, h0=h0, label=f"wg sums chunks {mode}")


def _degenerate(inp):
    """A = 0 for some states, delta = 0 at some steps, lambda exactly 0 and 1,
    theta = 0 for some states, mixed into ordinary inputs."""
    out = dict(inp)
    out["A"] = inp["A"].clone()
    out["A"][::3, 1::4] = 0.0
    out["delta"] = inp["delta"].clone()
    out["delta"][:, 5::17] = 0
    if inp["lam"] is not None:
        out["lam"] = inp["lam"].clone()
        out["lam"][:, ::11] = 0
        out["lam"][:, 3::11] = 1
    if inp["theta"] is not None:
        out["theta"] = inp["theta"].clone()
        out["theta"][..., ::5] = 0
    return out


@pytest.mark.parametrize("mode", ["real_zoh_f32", "real_trap_f32", "complex_trap_f32", "complex_trap_bf16"])
def test_backward_degenerate_values(mode):
    """Degenerate values (ZOH's dA at A = 0 comes from its series), D = 32 so
    the workgroup sums of dB and dC run."""
    w = MODES[mode].scaled(batch=2, dim=32, seqlen=150)
    inp = _degenerate(make_inputs(w, seed=28, device="cuda"))
    gen = torch.Generator(device="cuda").manual_seed(11)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    _compare(w, inp, dy, label=f"degenerate {mode}")


@pytest.mark.parametrize("N", [1, 33, 64])
def test_backward_state_sizes(N):
    w = MODES["complex_trap_f32"].scaled(batch=2, dim=6, seqlen=45, dstate=N)
    inp = make_inputs(w, seed=23, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda")
    _compare(w, inp, dy, label=f"N={N}")


def test_backward_without_optional_inputs():
    """theta = NULL (complex, no rotation) and D = NULL."""
    w = MODES["complex_euler_f32"].scaled(batch=2, dim=9, seqlen=40)
    inp = dict(make_inputs(w, seed=24, device="cuda"), theta=None, Dskip=None)
    gen = torch.Generator(device="cuda").manual_seed(6)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda")
    _compare(w, inp, dy, label="no theta, no D")


def test_backward_full_size_sampled():
    """The complex trapezoidal bf16 workload at full size (B=4, D=2560, L=8192,
    N=16), in the configuration bench.py --backward times, compared on a channel
    sample: every per-channel gradient (du, ddelta, dlambda, dtheta, the sampled
    channels' rows of dA and dD).  dB and dC sum over all 2560 channels, which the
    oracle cannot sample; the small-shape tests compare them in full."""
    from selective_state_space_42_amd.inputs import channel_sample

    w = WORKLOADS["complex_trap_bf16_b4_d2560_l8192_n16"]
    inp = make_inputs(w, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(2)
    dy = torch.randn(inp["u"].shape, generator=gen, device="cuda").to(inp["u"].dtype)
    g = ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["theta"], inp["lam"],
                     dy=dy, disc=w.disc)
    torch.cuda.synchronize()
    idx = sorted(np.random.default_rng(1).choice(w.dim, 6, replace=False).tolist())
    x = channel_sample(inp, idx)
    sel = torch.as_tensor(idx, device="cuda")
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                          disc=w.disc, is_complex=True, dy=_host(dy.index_select(2, sel)))
    errs = {
        "du": rel_err(_host(g["du"].index_select(2, sel)), ref["du"]),
        "ddelta": rel_err(_host(g["ddelta"].index_select(2, sel)), ref["ddelta"]),
        "dlambda": rel_err(_host(g["dlambda"].index_select(2, sel)), ref["dlambda"]),
        "dtheta": rel_err(_host(g["dtheta"].index_select(2, sel)), ref["dtheta"]),
        "dA": rel_err(_host(g["dA"].index_select(0, sel)), ref["dA"]),
        "dD": rel_err(_host(g["dD"].index_select(0, sel)), ref["dD"]),
    }
    print("backward full size " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) <= GRAD_TOL["bf16"], errs
