"""GPU parity of the SSD form (ssm_ssd_fwd) against the fp64 oracle.

The SSD setting (scalar A per head, one step size per (b, t, head), real state,
exponential-Euler b-terms) is the scan with delta and A broadcast over each
head's channels, so the oracle is the scan oracle run on that broadcast
problem (selective_state_space_42_amd.inputs.ssd_as_scan).  I/O is bf16, so
the bar is the scan's bf16 tolerance, 2e-2 (the intra-chunk matrix is also
rounded to bf16 for the MFMA units).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, rel_err
from selective_state_space_42_amd.inputs import SSD_WORKLOADS, make_ssd_inputs, ssd_as_scan
from selective_state_space_42_amd.scan import ssm_scan_fwd, ssm_ssd_fwd

pytestmark = pytest.mark.gpu

BASE = SSD_WORKLOADS["ssd_real_bf16_b4_d2560_l8192_n16_p64"]


def _host(t):
    return t.detach().float().cpu().double().numpy()


def _check(w, seed, d_index=None, label=""):
    inp = make_ssd_inputs(w, seed=seed, device="cuda")
    y, h = ssm_ssd_fwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], headdim=w.headdim)
    torch.cuda.synchronize()
    x = ssd_as_scan(inp, w, d_index)
    ref_y, ref_h = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], disc="euler",
                               is_complex=False)
    if d_index is not None:
        sel = torch.as_tensor(list(d_index), device="cuda")
        y, h = y.index_select(2, sel), h.index_select(1, sel)
    err_y, err_h = rel_err(_host(y), ref_y), rel_err(_host(h), ref_h)
    print(f"{label} err_y={err_y:.3e} err_h={err_h:.3e}", flush=True)
    assert err_y <= TOL["bf16"] and err_h <= TOL["bf16"], (err_y, err_h)
    return inp, y


@pytest.mark.parametrize("L", [1, 40, 64, 333])
def test_ssd_lengths(L):
    """One partial chunk, exactly one chunk, several chunks with a ragged tail."""
    _check(BASE.scaled(batch=2, dim=128, seqlen=L), seed=41, label=f"L={L}")


@pytest.mark.parametrize("N", [1, 5, 8, 24, 33, 40, 64])
def test_ssd_state_sizes(N):
    """N a multiple of 8 moves B, C and the chunk states in 16-byte pieces (24 and
    40 leave part of the last round of pieces unused); other N element by element."""
    _check(BASE.scaled(batch=2, dim=192, seqlen=150, dstate=N), seed=42, label=f"N={N}")


def test_ssd_unaligned_b_and_c_take_the_element_path():
    """B and C one element off 16-byte alignment take the element-by-element
    staging; its result is bit-identical to the 16-byte pieces' (both stage
    the same bf16 values)."""
    w = BASE.scaled(batch=2, dim=128, seqlen=333)
    inp = make_ssd_inputs(w, seed=44, device="cuda")

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        out = buf[1:].view(t.shape)
        out.copy_(t)
        return out

    args = (inp["u"], inp["delta"], inp["A"])
    y, h = ssm_ssd_fwd(*args, inp["Bm"], inp["Cm"], inp["Dskip"], headdim=w.headdim)
    y2, h2 = ssm_ssd_fwd(*args, shifted(inp["Bm"]), shifted(inp["Cm"]), inp["Dskip"], headdim=w.headdim)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(h, h2)


def test_ssd_matches_the_general_scan_kernel():
    """The same problem through ssm_scan_fwd (chunked scan kernel): both GPU paths agree."""
    w = BASE.scaled(batch=2, dim=128, seqlen=700)
    inp, y = _check(w, seed=43, label="vs scan")
    heads = torch.arange(w.dim, device="cuda") // w.headdim
    delta = inp["delta"].index_select(2, heads).contiguous()
    A = inp["A"].index_select(0, heads)[:, None].expand(w.dim, w.dstate).contiguous()
    y2, _ = ssm_scan_fwd(inp["u"], delta, A, inp["Bm"], inp["Cm"], inp["Dskip"], disc="euler")
    torch.cuda.synchronize()
    err = rel_err(_host(y), _host(y2))
    assert err <= TOL["bf16"], err


def test_ssd_full_size_sampled():
    """The SSD workload bench.py times (B=4, D=2560, L=8192, N=16, heads of 64),
    compared on a sample of channels (every batch row and step)."""
    idx = sorted(np.random.default_rng(3).choice(BASE.dim, 12, replace=False).tolist())
    _check(BASE, seed=None, d_index=idx, label="full size")


def test_ssd_degenerate_values():
    """A head with A = 0 (no decay: cum stays 0) and steps with delta = 0 (the
    state is held, nothing enters), over several chunks with a ragged tail."""
    w = BASE.scaled(batch=2, dim=192, seqlen=150)
    inp = dict(make_ssd_inputs(w, seed=46, device="cuda"))
    inp["A"] = inp["A"].clone()
    inp["A"][1] = 0.0
    inp["delta"] = inp["delta"].clone()
    inp["delta"][:, 7::13] = 0
    y, h = ssm_ssd_fwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], headdim=w.headdim)
    torch.cuda.synchronize()
    x = ssd_as_scan(inp, w)
    ref_y, ref_h = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], disc="euler",
                               is_complex=False)
    err_y, err_h = rel_err(_host(y), ref_y), rel_err(_host(h), ref_h)
    print(f"degenerate err_y={err_y:.3e} err_h={err_h:.3e}", flush=True)
    assert err_y <= TOL["bf16"] and err_h <= TOL["bf16"], (err_y, err_h)
