"""Thin Python binding of libssmscan.so (argument marshalling only).

The names mirror the C ABI in include/ssm_scan.h.  Every step of the scan runs
in the HIP kernels of the library; torch only provides device memory and the
stream.  There is no fallback: if the library is missing or its call fails,
these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIB names another build of the library (the sanitizer tests load a
# host-only AddressSanitizer/UBSan build of the argument checking through it)
LIB_PATH = os.environ.get("SSM_SCAN_LIB") or os.path.join(_PKG, "libssmscan.so")

SSM_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
SSM_DISC = {"zoh": 0, "euler": 1, "trap": 2}
SSM_ALGO = {"auto": 0, "sequential": 1, "chunked": 2, "sweep": 3}
ABI_VERSION = 5


class ScanDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("disc", ctypes.c_int32),
        ("is_complex", ctypes.c_int32), ("algo", ctypes.c_int32),
    ]


class SsdDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("headdim", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MimoDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64), ("chunk", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32), ("disc", ctypes.c_int32), ("is_complex", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class ScanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = ssm_scan_status_string(status)
        if status == 4:
            msg += f" (hipError_t {_lib().ssm_scan_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m selective_state_space_42_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)  # torch is imported first, so its HIP runtime is the one in use
    vp = ctypes.c_void_p
    lib.ssm_scan_fwd.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 11 + [ctypes.c_size_t, vp]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_ex.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 14 + [ctypes.c_size_t, vp]
    lib.ssm_scan_fwd_ex.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 11
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_calibrate_stream.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, ctypes.c_int32, vp, vp]
    lib.ssm_calibrate_stream.restype = ctypes.c_int
    lib.ssm_calibrate_device_math.argtypes = [ctypes.c_int32, vp, vp, vp, ctypes.c_int64, vp]
    lib.ssm_calibrate_device_math.restype = ctypes.c_int
    lib.ssm_scan_step.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 13
    lib.ssm_scan_step.restype = ctypes.c_int
    lib.ssm_scan_bwd.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 21 + [ctypes.c_size_t, vp]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ScanDesc)]
    lib.ssm_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_ssd_fwd.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 9 + [ctypes.c_size_t, vp]
    lib.ssm_ssd_fwd.restype = ctypes.c_int
    lib.ssm_ssd_workspace_bytes.argtypes = [ctypes.POINTER(SsdDesc)]
    lib.ssm_ssd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_mimo_fwd.argtypes = [ctypes.POINTER(MimoDesc)] + [vp] * 14 + [ctypes.c_size_t, vp]
    lib.ssm_mimo_fwd.restype = ctypes.c_int
    lib.ssm_mimo_step.argtypes = [ctypes.POINTER(MimoDesc)] + [vp] * 13
    lib.ssm_mimo_step.restype = ctypes.c_int
    lib.ssm_mimo_workspace_bytes.argtypes = [ctypes.POINTER(MimoDesc)]
    lib.ssm_mimo_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_algo.argtypes = [ctypes.POINTER(ScanDesc)]
    lib.ssm_scan_algo.restype = ctypes.c_int
    lib.ssm_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanDesc)]
    lib.ssm_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_status_string.argtypes = [ctypes.c_int]
    lib.ssm_scan_status_string.restype = ctypes.c_char_p
    lib.ssm_scan_abi_version.argtypes = []
    lib.ssm_scan_abi_version.restype = ctypes.c_int
    lib.ssm_scan_last_hip_error.argtypes = []
    lib.ssm_scan_last_hip_error.restype = ctypes.c_int
    if lib.ssm_scan_abi_version() != ABI_VERSION:
        raise RuntimeError("libssmscan.so ABI version mismatch")
    _LIB = lib
    return lib


def make_desc(batch, seqlen, dim, dstate, io_dtype, disc, is_complex, algo="auto") -> ScanDesc:
    return ScanDesc(int(batch), int(seqlen), int(dim), int(dstate), int(SSM_DTYPE.get(io_dtype, io_dtype)),
                    int(SSM_DISC.get(disc, disc)), int(bool(is_complex)), int(SSM_ALGO.get(algo, algo)))


def ssm_scan_abi_version() -> int:
    return _lib().ssm_scan_abi_version()


def ssm_scan_status_string(status: int) -> str:
    return _lib().ssm_scan_status_string(int(status)).decode()


def ssm_scan_algo(desc: ScanDesc) -> str:
    """Name of the kernel family ssm_scan_fwd runs for `desc` (AUTO resolved)."""
    v = int(_lib().ssm_scan_algo(ctypes.byref(desc)))
    if v < 0:
        raise ScanError(1, "ssm_scan_algo")
    return {a: k for k, a in SSM_ALGO.items()}[v]


def ssm_scan_workspace_bytes(desc: ScanDesc) -> int:
    return int(_lib().ssm_scan_workspace_bytes(ctypes.byref(desc)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_IO_DTYPES = (torch.float32, torch.bfloat16)


def _check(where: str, io_dtype, specs) -> None:
    """Argument checks done before any library call (validation, no arithmetic).

    `specs` lists (name, tensor or None, expected shape, expected dtype), with
    None as the dtype meaning the I/O dtype.  Every given tensor must be dense
    row-major (the library takes plain pointers with no strides), have exactly
    the expected shape and dtype, and live on the same GPU as the others.
    """
    if io_dtype not in _IO_DTYPES:
        raise ValueError(f"{where}: I/O dtype must be float32 or bfloat16, got {io_dtype}")
    device = None
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{where}: {name} must be a torch.Tensor")
        want = io_dtype if dtype is None else dtype
        if t.dtype != want:
            raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected {want}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous (dense row-major)")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{where}: {name} is on {t.device}, other arguments on {device}")
    if device is None or device.type != "cuda":
        raise ValueError(f"{where}: arguments must be GPU tensors (got {device})")


def _check_workspace(where: str, workspace, device) -> None:
    if workspace is None:
        return
    if workspace.device != device or not workspace.is_contiguous() or workspace.dim() != 1:
        raise ValueError(f"{where}: workspace must be a contiguous 1-D tensor on {device}")


def _dims(where: str, t, n: int, name: str):
    if not isinstance(t, torch.Tensor) or t.dim() != n:
        raise ValueError(f"{where}: {name} must be a {n}-D tensor")
    return tuple(t.shape)


def _scan_specs(where, u, delta, A, B, C, D, theta, lam, y, disc, is_complex):
    """Expected shapes of the scan's arguments (u, delta, lam, y (B,L,D); A
    (D,N); B, C (B,L,N) or (B,L,N,2); D (D,); theta (B,L,D,N)), for _check."""
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    bc = (Bsz, L, N, 2) if is_complex else (Bsz, L, N)
    if (disc == "trap") != (lam is not None):
        raise ValueError(f"{where}: lam is required for disc='trap' and only then")
    if theta is not None and not is_complex:
        raise ValueError(f"{where}: theta is only taken with a complex state")
    return [("u", u, (Bsz, L, Dm), None), ("delta", delta, (Bsz, L, Dm), None), ("A", A, (Dm, N), torch.float32),
            ("B", B, bc, None), ("C", C, bc, None), ("D", D, (Dm,), torch.float32),
            ("theta", theta, (Bsz, L, Dm, N), None), ("lam", lam, (Bsz, L, Dm), None), ("y", y, (Bsz, L, Dm), None)]


def ssm_scan_fwd(u, delta, A, B, C, D=None, theta=None, lam=None, *, disc: str, y=None, h_last=None,
                 want_h_last: bool = True, workspace=None, algo: str = "auto", stream=None):
    """Run the scan on torch device tensors; returns (y, h_last).

    Layouts as in include/ssm_scan.h: u, delta, lam (B,L,D); A (D,N) fp32;
    B, C (B,L,N) real or (B,L,N,2) complex; D (D,) fp32; theta (B,L,D,N).
    The state is complex when B has a trailing dimension of 2.  y, h_last and
    the workspace are allocated with torch when not given.
    """
    Bsz, L, Dm = _dims("ssm_scan_fwd", u, 3, "u")
    N = _dims("ssm_scan_fwd", A, 2, "A")[1]
    is_complex = B.dim() == 4
    specs = _scan_specs("ssm_scan_fwd", u, delta, A, B, C, D, theta, lam, y, disc, is_complex)
    shape = (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N)
    _check("ssm_scan_fwd", u.dtype, specs + [("h_last", h_last, shape, torch.float32)])
    desc = make_desc(Bsz, L, Dm, N, u.dtype, disc, is_complex, algo)
    _check_workspace("ssm_scan_fwd", workspace, u.device)
    if y is None:
        y = torch.empty_like(u)
    if h_last is None and want_h_last:
        h_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    need = ssm_scan_workspace_bytes(desc)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_scan_fwd(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(theta), _ptr(lam), _ptr(y), _ptr(h_last), _ptr(workspace), ws_bytes,
                             ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_scan_fwd")
    return y, h_last


def ssm_scan_fwd_ex(u, delta, A, B, C, D=None, theta=None, lam=None, h0=None, q0=None, *, disc: str, y=None,
                    h_last=None, q_last=None, want_h_last: bool = True, want_q_last: bool = False,
                    workspace=None, algo: str = "auto", stream=None):
    """Continuation of a scan; returns (y, h_last, q_last).

    As ssm_scan_fwd, plus h0 (the state before step 0) and, for the
    trapezoid, q0 = B_{-1} u_{-1}; both have the layout of h_last and may be
    None (zero).  q_last = B_{L-1} u_{L-1} is returned for the trapezoid when
    want_q_last (else None).
    """
    Bsz, L, Dm = _dims("ssm_scan_fwd_ex", u, 3, "u")
    N = _dims("ssm_scan_fwd_ex", A, 2, "A")[1]
    is_complex = B.dim() == 4
    specs = _scan_specs("ssm_scan_fwd_ex", u, delta, A, B, C, D, theta, lam, y, disc, is_complex)
    shape = (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N)
    if disc != "trap" and (q0 is not None or q_last is not None or want_q_last):
        raise ValueError("ssm_scan_fwd_ex: q0 and q_last belong to the trapezoid only")
    _check("ssm_scan_fwd_ex", u.dtype, specs + [("h0", h0, shape, torch.float32), ("q0", q0, shape, torch.float32),
                                                ("h_last", h_last, shape, torch.float32),
                                                ("q_last", q_last, shape, torch.float32)])
    _check_workspace("ssm_scan_fwd_ex", workspace, u.device)
    desc = make_desc(Bsz, L, Dm, N, u.dtype, disc, is_complex, algo)
    if y is None:
        y = torch.empty_like(u)
    if h_last is None and want_h_last:
        h_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    if q_last is None and want_q_last:
        q_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    need = ssm_scan_workspace_bytes(desc)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_scan_fwd_ex(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(theta), _ptr(lam), _ptr(h0), _ptr(q0), _ptr(y), _ptr(h_last), _ptr(q_last),
                                _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_scan_fwd_ex")
    return y, h_last, q_last


def ssm_scan_fwd_noalloc(u, delta, A, B, C, D=None, theta=None, lam=None, *, disc: str, y=None, h_last=None,
                         want_h_last: bool = True, algo: str = "auto", stream=None):
    """ssm_scan_fwd with the library's fixed per-GPU scratch instead of a
    workspace (the call allocates nothing; y and h_last are allocated here
    only when not given).  Returns (y, h_last)."""
    Bsz, L, Dm = _dims("ssm_scan_fwd_noalloc", u, 3, "u")
    N = _dims("ssm_scan_fwd_noalloc", A, 2, "A")[1]
    is_complex = B.dim() == 4
    specs = _scan_specs("ssm_scan_fwd_noalloc", u, delta, A, B, C, D, theta, lam, y, disc, is_complex)
    shape = (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N)
    _check("ssm_scan_fwd_noalloc", u.dtype, specs + [("h_last", h_last, shape, torch.float32)])
    desc = make_desc(Bsz, L, Dm, N, u.dtype, disc, is_complex, algo)
    if y is None:
        y = torch.empty_like(u)
    if h_last is None and want_h_last:
        h_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream
    st = _lib().ssm_scan_fwd_noalloc(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(theta), _ptr(lam), _ptr(y), _ptr(h_last), ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_scan_fwd_noalloc")
    return y, h_last


def ssm_calibrate_stream(src, dst, nontemporal: bool = False, clocks=None, stream=None) -> None:
    """Enqueue the library's read-dominant stream kernel: reads all of `src`,
    writes all of `dst` (contiguous GPU tensors; src bytes an integer multiple,
    1 to 64, of dst bytes).  `clocks`, a GPU int64 tensor of 2, receives the
    shader-clock and 100 MHz real-time ticks of the run."""
    for name, t in (("src", src), ("dst", dst)):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"ssm_calibrate_stream: {name} must be a contiguous GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    st = _lib().ssm_calibrate_stream(_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                     dst.numel() * dst.element_size(), int(bool(nontemporal)), _ptr(clocks),
                                     ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_calibrate_stream")


DEVICE_MATH = {"exp_dA": 0, "sin_hw": 1, "cos_hw": 2, "sin_poly": 3, "cos_poly": 4, "sin_wide": 5, "cos_wide": 6,
               "expm1_zoh": 7, "exp_zoh": 8}


def ssm_calibrate_device_math(fn: str, x, y=None, out=None, stream=None):
    """The scan kernel's transcendental policy `fn` (a key of DEVICE_MATH)
    applied element-wise on the GPU: out[i] = f(x[i], y[i]) (fp32 GPU tensors
    of one shape; y for exp_dA, expm1_zoh and exp_zoh only)."""
    code = DEVICE_MATH[fn]
    needs_y = code == 0 or code >= 7
    ts = [("x", x)] + ([("y", y)] if needs_y else [])
    for name, t in ts:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous() \
                or t.device.type != "cuda":
            raise ValueError(f"ssm_calibrate_device_math: {name} must be a contiguous fp32 GPU tensor")
    if needs_y and y.shape != x.shape:
        raise ValueError("ssm_calibrate_device_math: y must have x's shape")
    if out is None:
        out = torch.empty_like(x)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = _lib().ssm_calibrate_device_math(code, _ptr(x), _ptr(y) if needs_y else None, _ptr(out), x.numel(),
                                          ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_calibrate_device_math")
    return out


def ssm_scan_step(u, delta, A, B, C, D=None, theta=None, lam=None, *, h, u_prev=None, B_prev=None, disc: str,
                  y=None, stream=None):
    """One decode step, updating h in place; returns y.

    u, delta, lam, u_prev (B,D); A (D,N) fp32; B, C, B_prev (B,N) real or
    (B,N,2) complex; D (D,) fp32; theta (B,D,N); h (B,D,N) or (B,D,N,2) fp32.
    u_prev and B_prev (the previous step's u and B) are for the trapezoid.
    """
    Bsz, Dm = _dims("ssm_scan_step", u, 2, "u")
    N = _dims("ssm_scan_step", A, 2, "A")[1]
    is_complex = B.dim() == 3
    bc = (Bsz, N, 2) if is_complex else (Bsz, N)
    if (disc == "trap") != (lam is not None):
        raise ValueError("ssm_scan_step: lam is required for disc='trap' and only then")
    if (u_prev is None) != (B_prev is None) or (disc != "trap" and u_prev is not None):
        raise ValueError("ssm_scan_step: u_prev and B_prev go together, for the trapezoid only")
    if theta is not None and not is_complex:
        raise ValueError("ssm_scan_step: theta is only taken with a complex state")
    _check("ssm_scan_step", u.dtype, [
        ("u", u, (Bsz, Dm), None), ("delta", delta, (Bsz, Dm), None), ("A", A, (Dm, N), torch.float32),
        ("B", B, bc, None), ("C", C, bc, None), ("D", D, (Dm,), torch.float32), ("theta", theta, (Bsz, Dm, N), None),
        ("lam", lam, (Bsz, Dm), None), ("u_prev", u_prev, (Bsz, Dm), None), ("B_prev", B_prev, bc, None),
        ("h", h, (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N), torch.float32), ("y", y, (Bsz, Dm), None)])
    desc = make_desc(Bsz, 1, Dm, N, u.dtype, disc, is_complex)
    if y is None:
        y = torch.empty_like(u)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_scan_step(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                              _ptr(theta), _ptr(lam), _ptr(u_prev), _ptr(B_prev), _ptr(h), _ptr(y),
                              ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_scan_step")
    return y


def ssm_scan_bwd_workspace_bytes(desc: ScanDesc) -> int:
    return int(_lib().ssm_scan_bwd_workspace_bytes(ctypes.byref(desc)))


def ssm_scan_bwd(u, delta, A, B, C, D=None, theta=None, lam=None, h0=None, *, dy, dh_last=None, disc: str,
                 want_dD: bool = True, want_dtheta: bool = True, want_dh0: bool = False, workspace=None,
                 stream=None) -> dict:
    """Gradients of sum(dy * y) + <dh_last, h_last>; returns a dict of fp32 tensors
    du, ddelta, dA, dB, dC, dD, dtheta, dlambda, dh0 (None where not computed)."""
    Bsz, L, Dm = _dims("ssm_scan_bwd", u, 3, "u")
    N = _dims("ssm_scan_bwd", A, 2, "A")[1]
    is_complex = B.dim() == 4
    specs = _scan_specs("ssm_scan_bwd", u, delta, A, B, C, D, theta, lam, None, disc, is_complex)
    hshape = (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N)
    if dy is None:
        raise ValueError("ssm_scan_bwd: dy is required")
    _check("ssm_scan_bwd", u.dtype, specs + [("dy", dy, (Bsz, L, Dm), None), ("h0", h0, hshape, torch.float32),
                                             ("dh_last", dh_last, hshape, torch.float32)])
    _check_workspace("ssm_scan_bwd", workspace, u.device)
    desc = make_desc(Bsz, L, Dm, N, u.dtype, disc, is_complex)
    f32 = dict(dtype=torch.float32, device=u.device)
    g = dict(du=torch.empty((Bsz, L, Dm), **f32), ddelta=torch.empty((Bsz, L, Dm), **f32),
             dA=torch.empty((Dm, N), **f32), dB=torch.empty(B.shape, **f32), dC=torch.empty(C.shape, **f32),
             dD=torch.empty((Dm,), **f32) if want_dD else None,
             dtheta=torch.empty(theta.shape, **f32) if (theta is not None and want_dtheta) else None,
             dlambda=torch.empty((Bsz, L, Dm), **f32) if disc == "trap" else None,
             dh0=torch.empty(hshape, **f32) if want_dh0 else None)
    need = ssm_scan_bwd_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_scan_bwd(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(theta), _ptr(lam), _ptr(h0), _ptr(dy), _ptr(dh_last),
                             *(_ptr(g[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dtheta", "dlambda",
                                                    "dh0")),
                             _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_scan_bwd")
    return g


def make_ssd_desc(batch, seqlen, dim, dstate, headdim, io_dtype) -> SsdDesc:
    return SsdDesc(int(batch), int(seqlen), int(dim), int(dstate), int(headdim),
                   int(SSM_DTYPE.get(io_dtype, io_dtype)), 0)


def ssm_ssd_workspace_bytes(desc: SsdDesc) -> int:
    return int(_lib().ssm_ssd_workspace_bytes(ctypes.byref(desc)))


def ssm_ssd_fwd(u, delta, A, B, C, D=None, *, headdim: int = 64, y=None, h_last=None, want_h_last: bool = True,
                workspace=None, stream=None):
    """The SSD form on torch device tensors; returns (y, h_last).

    u (B,L,D) bf16; delta (B,L,H) bf16 with H = D / headdim; A (H,) fp32;
    B, C (B,L,N) bf16; D (D,) fp32.
    """
    Bsz, L, Dm = _dims("ssm_ssd_fwd", u, 3, "u")
    N = _dims("ssm_ssd_fwd", B, 3, "B")[2]
    if headdim < 1 or Dm % headdim:
        raise ValueError(f"ssm_ssd_fwd: the channel count {Dm} is not a multiple of headdim {headdim}")
    H = Dm // headdim
    _check("ssm_ssd_fwd", u.dtype, [
        ("u", u, (Bsz, L, Dm), None), ("delta", delta, (Bsz, L, H), None), ("A", A, (H,), torch.float32),
        ("B", B, (Bsz, L, N), None), ("C", C, (Bsz, L, N), None), ("D", D, (Dm,), torch.float32),
        ("y", y, (Bsz, L, Dm), None), ("h_last", h_last, (Bsz, Dm, N), torch.float32)])
    _check_workspace("ssm_ssd_fwd", workspace, u.device)
    desc = make_ssd_desc(Bsz, L, Dm, N, headdim, u.dtype)
    if y is None:
        y = torch.empty_like(u)
    if h_last is None and want_h_last:
        h_last = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=u.device)
    need = ssm_ssd_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_ssd_fwd(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                            _ptr(h_last), _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_ssd_fwd")
    return y, h_last


def make_mimo_desc(batch, seqlen, dim, dstate, rank, io_dtype, disc, is_complex, chunk: int = 0) -> MimoDesc:
    return MimoDesc(int(batch), int(seqlen), int(dim), int(dstate), int(rank), int(chunk),
                    int(SSM_DTYPE.get(io_dtype, io_dtype)), int(SSM_DISC.get(disc, disc)), int(bool(is_complex)), 0)


def ssm_mimo_workspace_bytes(desc: MimoDesc) -> int:
    return int(_lib().ssm_mimo_workspace_bytes(ctypes.byref(desc)))


def ssm_mimo_fwd(u, delta, A, B, C, D=None, theta=None, lam=None, h0=None, q0=None, *, disc: str, y=None,
                 h_last=None, q_last=None, want_h_last: bool = True, want_q_last: bool = False, workspace=None,
                 chunk: int = 0, stream=None):
    """The MIMO scan on torch device tensors; returns (y, h_last, q_last).

    u (B,L,D,R); delta, lam (B,L,D); A (D,N) fp32; B, C (B,L,N,R) real or
    (B,L,N,R,2) complex; D (D,) fp32; theta (B,L,D,N); h0, q0 and the
    returned states (B,D,N[,2]) fp32.  chunk fixes the time-chunk length
    (0: the library's choice).
    """
    Bsz, L, Dm, R = _dims("ssm_mimo_fwd", u, 4, "u")
    N = _dims("ssm_mimo_fwd", A, 2, "A")[1]
    is_complex = B.dim() == 5
    shape = (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N)
    bc = (Bsz, L, N, R, 2) if is_complex else (Bsz, L, N, R)
    if (disc == "trap") != (lam is not None):
        raise ValueError("ssm_mimo_fwd: lam is required for disc='trap' and only then")
    if disc != "trap" and (q0 is not None or q_last is not None or want_q_last):
        raise ValueError("ssm_mimo_fwd: q0 and q_last belong to the trapezoid only")
    if theta is not None and not is_complex:
        raise ValueError("ssm_mimo_fwd: theta is only taken with a complex state")
    _check("ssm_mimo_fwd", u.dtype, [
        ("u", u, (Bsz, L, Dm, R), None), ("delta", delta, (Bsz, L, Dm), None), ("A", A, (Dm, N), torch.float32),
        ("B", B, bc, None), ("C", C, bc, None), ("D", D, (Dm,), torch.float32),
        ("theta", theta, (Bsz, L, Dm, N), None), ("lam", lam, (Bsz, L, Dm), None),
        ("h0", h0, shape, torch.float32), ("q0", q0, shape, torch.float32), ("y", y, (Bsz, L, Dm, R), None),
        ("h_last", h_last, shape, torch.float32), ("q_last", q_last, shape, torch.float32)])
    _check_workspace("ssm_mimo_fwd", workspace, u.device)
    desc = make_mimo_desc(Bsz, L, Dm, N, R, u.dtype, disc, is_complex, chunk)
    if y is None:
        y = torch.empty_like(u)
    if h_last is None and want_h_last:
        h_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    if q_last is None and want_q_last:
        q_last = torch.empty(shape, dtype=torch.float32, device=u.device)
    need = ssm_mimo_workspace_bytes(desc)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_mimo_fwd(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(theta), _ptr(lam), _ptr(h0), _ptr(q0), _ptr(y), _ptr(h_last), _ptr(q_last),
                             _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_mimo_fwd")
    return y, h_last, q_last


def ssm_mimo_step(u, delta, A, B, C, D=None, theta=None, lam=None, *, h, u_prev=None, B_prev=None, disc: str,
                  y=None, stream=None):
    """One MIMO decode step, updating h in place; returns y.

    u, u_prev (B,D,R); delta, lam (B,D); A (D,N) fp32; B, C, B_prev (B,N,R)
    real or (B,N,R,2) complex; D (D,) fp32; theta (B,D,N); h (B,D,N[,2]) fp32.
    """
    Bsz, Dm, R = _dims("ssm_mimo_step", u, 3, "u")
    N = _dims("ssm_mimo_step", A, 2, "A")[1]
    is_complex = B.dim() == 4
    bc = (Bsz, N, R, 2) if is_complex else (Bsz, N, R)
    if (disc == "trap") != (lam is not None):
        raise ValueError("ssm_mimo_step: lam is required for disc='trap' and only then")
    if (u_prev is None) != (B_prev is None) or (disc != "trap" and u_prev is not None):
        raise ValueError("ssm_mimo_step: u_prev and B_prev go together, for the trapezoid only")
    if theta is not None and not is_complex:
        raise ValueError("ssm_mimo_step: theta is only taken with a complex state")
    _check("ssm_mimo_step", u.dtype, [
        ("u", u, (Bsz, Dm, R), None), ("delta", delta, (Bsz, Dm), None), ("A", A, (Dm, N), torch.float32),
        ("B", B, bc, None), ("C", C, bc, None), ("D", D, (Dm,), torch.float32), ("theta", theta, (Bsz, Dm, N), None),
        ("lam", lam, (Bsz, Dm), None), ("u_prev", u_prev, (Bsz, Dm, R), None), ("B_prev", B_prev, bc, None),
        ("h", h, (Bsz, Dm, N, 2) if is_complex else (Bsz, Dm, N), torch.float32), ("y", y, (Bsz, Dm, R), None)])
    desc = make_mimo_desc(Bsz, 1, Dm, N, R, u.dtype, disc, is_complex)
    if y is None:
        y = torch.empty_like(u)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream if u.is_cuda else 0
    st = _lib().ssm_mimo_step(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                              _ptr(theta), _ptr(lam), _ptr(u_prev), _ptr(B_prev), _ptr(h), _ptr(y),
                              ctypes.c_void_p(stream))
    if st != 0:
        raise ScanError(st, "ssm_mimo_step")
    return y
