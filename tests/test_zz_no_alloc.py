"""GPU test of ssm_scan_fwd_noalloc, the entry point that allocates nothing.

It runs the chunked kernels of ssm_scan_fwd with the library's fixed per-GPU
scratch buffer in place of a caller workspace.  Two calls in a row, the
second on a smaller problem (so the buffer holds the first call's flags and
payloads when the second starts), are each compared with ssm_scan_fwd on the
same inputs and with the fp64 oracle, at the scan's tolerances (1e-5 for fp32
I/O, 2e-2 for bf16 I/O).  The call goes through the C ABI with ctypes.
"""
import ctypes

import pytest
import torch

from parity_util import TOL, oracle_for, rel_err, rel_err_complex
from selective_state_space_42_amd import scan
from selective_state_space_42_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20
_TRAP = WORKLOADS["complex_trap_bf16_b4_d2560_l8192_n16"]
_EULER = WORKLOADS["complex_euler_b8_d2048_l4096_n16"]
_ZOH = WORKLOADS["real_zoh_b8_d1536_l2048_n16"]


def _noalloc(inputs, w, y, h_last):
    desc = scan.make_desc(w.batch, w.seqlen, w.dim, w.dstate, inputs["u"].dtype, w.disc, w.is_complex, "chunked")
    p = scan._ptr
    st = scan._lib().ssm_scan_fwd_noalloc(
        ctypes.byref(desc), p(inputs["u"]), p(inputs["delta"]), p(inputs["A"]), p(inputs["Bm"]), p(inputs["Cm"]),
        p(inputs["Dskip"]), p(inputs["theta"]), p(inputs["lam"]), p(y), p(h_last),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, desc


def _check_case(w, seed):
    inputs = make_inputs(w, seed, device="cuda")
    desc = scan.make_desc(w.batch, w.seqlen, w.dim, w.dstate, inputs["u"].dtype, w.disc, w.is_complex, "chunked")
    need = scan.ssm_scan_workspace_bytes(desc)
    assert 0 < need <= SCRATCH_BYTES, need
    y = torch.empty_like(inputs["u"])
    h = torch.empty((w.batch, w.dim, w.dstate, 2) if w.is_complex else (w.batch, w.dim, w.dstate),
                    dtype=torch.float32, device="cuda")
    print(f"noalloc {w.name} seed {seed} (workspace {need} bytes)", flush=True)
    st, _ = _noalloc(inputs, w, y, h)
    assert st == 0, scan.ssm_scan_status_string(st)
    y_ref, h_ref = scan.ssm_scan_fwd(inputs["u"], inputs["delta"], inputs["A"], inputs["Bm"], inputs["Cm"],
                                     inputs["Dskip"], inputs["theta"], inputs["lam"], disc=w.disc, algo="chunked")
    torch.cuda.synchronize()
    tol = TOL[w.io_dtype]
    hc = rel_err_complex if w.is_complex else rel_err
    e_y = rel_err(y.float().cpu().double().numpy(), y_ref.float().cpu().double().numpy())
    e_h = hc(h.cpu().double().numpy(), h_ref.cpu().double().numpy())
    d_index = list(range(0, w.dim, max(1, w.dim // 8)))
    yo, ho = oracle_for(inputs, w.disc, w.is_complex, d_index)
    idx = torch.as_tensor(d_index, device="cuda")
    e_yo = rel_err(y.index_select(2, idx).float().cpu().double().numpy(), yo)
    e_ho = hc(h.index_select(1, idx).cpu().double().numpy(), ho)
    print(f"  vs ssm_scan_fwd err_y={e_y:.3e} err_h={e_h:.3e}; vs oracle err_y={e_yo:.3e} err_h={e_ho:.3e}",
          flush=True)
    assert e_y <= tol and e_h <= tol and e_yo <= tol and e_ho <= tol, (e_y, e_h, e_yo, e_ho)


@pytest.mark.parametrize("base,first,second", [
    (_TRAP, dict(batch=2, dim=40, seqlen=3000), dict(batch=1, dim=16, seqlen=500)),
    (_EULER, dict(batch=2, dim=24, seqlen=2100), dict(batch=1, dim=9, seqlen=333)),
    (_ZOH, dict(batch=3, dim=32, seqlen=1000), dict(batch=1, dim=5, seqlen=97)),
])
def test_noalloc_matches_fwd_on_two_calls(base, first, second):
    _check_case(base.scaled(name=base.name + "_first", **first), seed=11)
    _check_case(base.scaled(name=base.name + "_second", **second), seed=12)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    w = _TRAP.scaled(batch=1, dim=1024, seqlen=1 << 17)
    desc = scan.make_desc(w.batch, w.seqlen, w.dim, w.dstate, torch.bfloat16, w.disc, True, "chunked")
    assert scan.ssm_scan_workspace_bytes(desc) > SCRATCH_BYTES
    small = _TRAP.scaled(batch=1, dim=8, seqlen=8)
    inputs = make_inputs(small, 3, device="cuda")   # pointers only; the call is rejected before any launch
    st, _ = _noalloc(inputs, w, inputs["u"], None)
    assert st == 5, scan.ssm_scan_status_string(st)
