"""The Python binding rejects malformed tensors before any library call.

The C ABI takes plain pointers to dense row-major buffers, so a strided view,
a wrong dtype or a wrong shape would make a kernel read the wrong elements or
past the end of a buffer.  These checks run on CPU tensors with the library
call replaced by a trap: every case must raise ValueError without reaching it.
"""
import pytest
import torch

from selective_state_space_42_amd import scan


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def trap():
        raise AssertionError("the library was called")
    monkeypatch.setattr(scan, "_lib", trap)


def scan_args(B=2, L=5, D=3, N=4, dtype=torch.bfloat16, cplx=True, trap=True):
    f32 = torch.float32
    a = dict(u=torch.zeros(B, L, D, dtype=dtype), delta=torch.zeros(B, L, D, dtype=dtype),
             A=torch.zeros(D, N, dtype=f32),
             B=torch.zeros((B, L, N, 2) if cplx else (B, L, N), dtype=dtype),
             C=torch.zeros((B, L, N, 2) if cplx else (B, L, N), dtype=dtype),
             D=torch.zeros(D, dtype=f32),
             theta=torch.zeros(B, L, D, N, dtype=dtype) if cplx else None,
             lam=torch.zeros(B, L, D, dtype=dtype) if trap else None)
    return a


def call_fwd(a, **kw):
    return scan.ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["theta"], a["lam"],
                             disc=kw.pop("disc", "trap" if a["lam"] is not None else "euler"), **kw)


def test_valid_cpu_tensors_stop_at_the_device_check():
    with pytest.raises(ValueError, match="GPU tensors"):
        call_fwd(scan_args())


@pytest.mark.parametrize("name", ["u", "delta", "B", "C", "theta", "lam"])
def test_io_dtype_mismatch(name):
    a = scan_args()
    a[name] = a[name].float()
    with pytest.raises(ValueError, match="dtype"):
        call_fwd(a)


@pytest.mark.parametrize("name", ["A", "D"])
def test_fp32_parameters(name):
    a = scan_args()
    a[name] = a[name].to(torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        call_fwd(a)


def test_unsupported_io_dtype():
    a = scan_args(dtype=torch.float16)
    with pytest.raises(ValueError, match="float32 or bfloat16"):
        call_fwd(a)


@pytest.mark.parametrize("name,shape", [
    ("delta", (2, 5, 4)), ("A", (3, 5)), ("B", (2, 5, 3, 2)), ("C", (2, 4, 4, 2)), ("D", (4,)),
    ("theta", (2, 5, 3, 3)), ("lam", (1, 5, 3))])
def test_shape_mismatch(name, shape):
    a = scan_args()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match="shape"):
        call_fwd(a)


@pytest.mark.parametrize("name", ["u", "theta", "B"])
def test_strided_views_rejected(name):
    a = scan_args()
    t = a[name]
    wide = torch.zeros(t.shape[:-1] + (2 * t.shape[-1],), dtype=t.dtype)
    a[name] = wide[..., ::2]
    assert a[name].shape == t.shape and not a[name].is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        call_fwd(a)


def test_transposed_view_rejected():
    a = scan_args(B=2, L=3, D=3)
    a["u"] = a["u"].transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        call_fwd(a)


def test_lambda_and_theta_rules():
    a = scan_args(trap=False)
    with pytest.raises(ValueError, match="lam"):
        call_fwd(a, disc="trap")
    a = scan_args(trap=True)
    with pytest.raises(ValueError, match="lam"):
        call_fwd(a, disc="euler")
    a = scan_args(cplx=False, trap=False)
    a["theta"] = torch.zeros(2, 5, 3, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="theta"):
        call_fwd(a, disc="euler")


def test_output_buffers_checked():
    a = scan_args()
    with pytest.raises(ValueError, match="y"):
        call_fwd(a, y=torch.zeros(2, 5, 3, dtype=torch.float32))
    with pytest.raises(ValueError, match="h_last"):
        call_fwd(a, h_last=torch.zeros(2, 3, 4, dtype=torch.float32))  # complex state needs (B, D, N, 2)


def test_continuation_states_checked():
    a = scan_args()
    with pytest.raises(ValueError, match="h0"):
        scan.ssm_scan_fwd_ex(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["theta"], a["lam"],
                             h0=torch.zeros(2, 3, 4, 2, dtype=torch.bfloat16), disc="trap")
    b = scan_args(trap=False)
    with pytest.raises(ValueError, match="trapezoid"):
        scan.ssm_scan_fwd_ex(b["u"], b["delta"], b["A"], b["B"], b["C"], b["D"], b["theta"], None,
                             q0=torch.zeros(2, 3, 4, 2), disc="euler")


def test_step_checks():
    f32 = torch.float32
    B, D, N = 2, 3, 4
    args = dict(u=torch.zeros(B, D), delta=torch.zeros(B, D), A=torch.zeros(D, N), B=torch.zeros(B, N, 2),
                C=torch.zeros(B, N, 2), D=None, theta=torch.zeros(B, D, N), lam=None)
    with pytest.raises(ValueError, match="h"):
        scan.ssm_scan_step(**args, h=torch.zeros(B, D, N, dtype=f32), disc="euler")
    with pytest.raises(ValueError, match="GPU"):
        scan.ssm_scan_step(**args, h=torch.zeros(B, D, N, 2, dtype=f32), disc="euler")
    with pytest.raises(ValueError, match="u_prev"):
        scan.ssm_scan_step(**args, h=torch.zeros(B, D, N, 2), u_prev=torch.zeros(B, D), disc="euler")


def test_backward_checks():
    a = scan_args()
    with pytest.raises(ValueError, match="dy"):
        scan.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["theta"], a["lam"],
                          dy=torch.zeros(2, 5, 3, dtype=torch.float32), disc="trap")


def test_ssd_checks():
    bf = torch.bfloat16
    u = torch.zeros(1, 8, 128, dtype=bf)
    ok = dict(delta=torch.zeros(1, 8, 2, dtype=bf), A=torch.zeros(2), B=torch.zeros(1, 8, 16, dtype=bf),
              C=torch.zeros(1, 8, 16, dtype=bf))
    with pytest.raises(ValueError, match="GPU"):
        scan.ssm_ssd_fwd(u, **ok)
    with pytest.raises(ValueError, match="shape"):
        scan.ssm_ssd_fwd(u, **{**ok, "delta": torch.zeros(1, 8, 128, dtype=bf)})
    with pytest.raises(ValueError, match="multiple"):
        scan.ssm_ssd_fwd(torch.zeros(1, 8, 100, dtype=bf), **ok)


def test_mimo_checks():
    bf = torch.bfloat16
    B, L, D, N, R = 1, 4, 3, 4, 2
    ok = dict(delta=torch.zeros(B, L, D, dtype=bf), A=torch.zeros(D, N), B=torch.zeros(B, L, N, R, 2, dtype=bf),
              C=torch.zeros(B, L, N, R, 2, dtype=bf), theta=torch.zeros(B, L, D, N, dtype=bf))
    u = torch.zeros(B, L, D, R, dtype=bf)
    with pytest.raises(ValueError, match="GPU"):
        scan.ssm_mimo_fwd(u, **ok, disc="euler")
    with pytest.raises(ValueError, match="shape"):
        scan.ssm_mimo_fwd(u, **{**ok, "C": torch.zeros(B, L, N, 2 * R, 2, dtype=bf)}, disc="euler")
    with pytest.raises(ValueError, match="dtype"):
        scan.ssm_mimo_fwd(u.float(), **ok, disc="euler")
    hs = torch.zeros(B, D, N, 2)
    with pytest.raises(ValueError, match="GPU"):
        scan.ssm_mimo_step(torch.zeros(B, D, R, dtype=bf), torch.zeros(B, D, dtype=bf), ok["A"],
                           torch.zeros(B, N, R, 2, dtype=bf), torch.zeros(B, N, R, 2, dtype=bf),
                           theta=torch.zeros(B, D, N, dtype=bf), h=hs, disc="euler")
