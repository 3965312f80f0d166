"""fp64 CPU oracle for the forward selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it (the oracle is plain C compiled with gcc, see
``ssm_oracle.c``; this file only marshals numpy arrays into it).

Functions:
  build()    -- compile ssm_oracle.c into liboracle.so with gcc (no fast-math,
                no FMA contraction).
  scan(...)  -- the sequential recurrence in fp64 (see ssm_oracle.c for the
                definition and the page sections it follows).
  combine()  -- the operator combine (a2,b2)(x)(a1,b1) = (a2 a1, a2 b1 + b2)
                from fengwang.github.io "complex parallel scan", section "the
                mathematical essence of the parallel scan".
  scan_bwd() -- gradients of the scan by reverse mode of the same sequential
                definition (ssm_oracle_bwd.c).
  scan_mimo() -- the multi-input multi-output form: R inputs and R outputs
                per token and channel sharing one state (ssm_oracle_mimo.c).

Parity status: every function here is pinned -- scan() and combine() by
tests/test_oracle_pins.py against closed forms, special cases and invariants,
scan_bwd() by tests/test_oracle_bwd_pins.py against central finite
differences of scan(), scan_mimo() by tests/test_oracle_mimo_pins.py against
scan() (R = 1 and superposition over the inputs) and a cumulative-sum closed
form; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_SRC_BWD = os.path.join(_HERE, "ssm_oracle_bwd.c")
_SRC_MIMO = os.path.join(_HERE, "ssm_oracle_mimo.c")
_SOURCES = (_SRC, _SRC_BWD, _SRC_MIMO)
_LIB = os.path.join(_HERE, "liboracle.so")

DISC = {"zoh": 0, "euler": 1, "trap": 2}

_lib = None


def build() -> str:
    """Compile the oracle with gcc.  Returns the path of the shared library."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
        "-ffp-contract=off", "-pthread", "-o", _LIB, *_SOURCES, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # SSM_ORACLE_LIB names another build of the same sources (the sanitizer
    # tests load an AddressSanitizer/UBSan build through it)
    path = os.environ.get("SSM_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(f) for f in _SOURCES):
            build()
    lib = ctypes.CDLL(path)
    dp = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_scan_f64.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int] + [dp] * 13 + [ctypes.c_int]
    lib.oracle_scan_f64.restype = ctypes.c_int
    lib.oracle_scan_bwd_f64.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int] + [dp] * 20
    lib.oracle_scan_bwd_f64.restype = ctypes.c_int
    lib.oracle_scan_mimo_f64.argtypes = [i64] * 5 + [ctypes.c_int, ctypes.c_int] + [dp] * 13 + [ctypes.c_int]
    lib.oracle_scan_mimo_f64.restype = ctypes.c_int
    lib.oracle_combine_f64.argtypes = [i64, dp, dp, dp, dp, dp, dp]
    lib.oracle_combine_f64.restype = None
    _lib = lib
    return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(u, delta, A, Bm, Cm, Dskip=None, theta=None, lam=None, *, disc: str, is_complex: bool,
         h0=None, q0=None, nthreads: int = 0, return_q: bool = False):
    """Run the fp64 oracle.

    Shapes (row-major): u, delta, lam: (B,L,D); A: (D,N); Bm, Cm: (B,L,N) real
    or (B,L,N,2) complex; Dskip: (D,); theta: (B,L,D,N).  h0/q0 optionally give
    the state and the previous step's q = Bm*u to continue from, with the
    layout of h_last.  Returns (y (B,L,D), h_last (B,D,N[,2])) and q_last when
    return_q is set.  Inputs are widened to fp64 (exact for fp32/bf16 values).
    """
    lib = _load()
    u, delta, A, Bm, Cm = map(_f64, (u, delta, A, Bm, Cm))
    Dskip, theta, lam, h0, q0 = map(_f64, (Dskip, theta, lam, h0, q0))
    B, L, D = u.shape
    N = A.shape[1]
    cw = (2,) if is_complex else ()
    y = np.empty((B, L, D), dtype=np.float64)
    h_last = np.empty((B, D, N) + cw, dtype=np.float64)
    q_last = np.empty((B, D, N) + cw, dtype=np.float64)
    rc = lib.oracle_scan_f64(
        B, L, D, N, DISC[disc], int(bool(is_complex)),
        _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(theta), _ptr(lam),
        _ptr(h0), _ptr(q0), _ptr(y), _ptr(h_last), _ptr(q_last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_f64 returned {rc}")
    if return_q:
        return y, h_last, q_last
    return y, h_last


def scan_bwd(u, delta, A, Bm, Cm, Dskip=None, theta=None, lam=None, *, disc: str, is_complex: bool,
             dy, dh_last=None, h0=None):
    """Gradients of L = sum(dy * y) + <dh_last, h_last> w.r.t. every input.

    Returns a dict with du, ddelta (B,L,D); dA (D,N); dB, dC (layout of Bm);
    dD (D,) when Dskip is given; dtheta (B,L,D,N) when theta is given;
    dlambda (B,L,D) for the trapezoid; dh0 (layout of h_last).  Complex
    gradients are (d/dre, d/dim).
    """
    lib = _load()
    u, delta, A, Bm, Cm, dy = map(_f64, (u, delta, A, Bm, Cm, dy))
    Dskip, theta, lam, h0, dh_last = map(_f64, (Dskip, theta, lam, h0, dh_last))
    B, L, D = u.shape
    N = A.shape[1]
    cw = (2,) if is_complex else ()
    out = dict(du=np.empty((B, L, D)), ddelta=np.empty((B, L, D)), dA=np.empty((D, N)),
               dB=np.empty(Bm.shape), dC=np.empty(Cm.shape),
               dD=np.empty((D,)) if Dskip is not None else None,
               dtheta=np.empty((B, L, D, N)) if theta is not None else None,
               dlambda=np.empty((B, L, D)) if disc == "trap" else None,
               dh0=np.empty((B, D, N) + cw))
    rc = lib.oracle_scan_bwd_f64(
        B, L, D, N, DISC[disc], int(bool(is_complex)),
        _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(theta), _ptr(lam), _ptr(h0),
        _ptr(dy), _ptr(dh_last), *(_ptr(out[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dtheta",
                                                          "dlambda", "dh0")))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd_f64 returned {rc}")
    return out


def scan_mimo(u, delta, A, Bm, Cm, Dskip=None, theta=None, lam=None, *, disc: str, is_complex: bool,
              h0=None, q0=None, nthreads: int = 0, return_q: bool = False):
    """The MIMO scan in fp64: one state per (b, d) shared by R inputs and outputs.

    Shapes (row-major): u: (B,L,D,R); delta, lam: (B,L,D); A: (D,N);
    Bm, Cm: (B,L,N,R) real or (B,L,N,R,2) complex; Dskip: (D,);
    theta: (B,L,D,N); h0, q0: layout of h_last.  Returns (y (B,L,D,R),
    h_last (B,D,N[,2])) and q_last (the trapezoid's q_{L-1} = sum_r B u)
    when return_q is set.
    """
    lib = _load()
    u, delta, A, Bm, Cm = map(_f64, (u, delta, A, Bm, Cm))
    Dskip, theta, lam, h0, q0 = map(_f64, (Dskip, theta, lam, h0, q0))
    B, L, D, R = u.shape
    N = A.shape[1]
    cw = (2,) if is_complex else ()
    if Bm.shape != (B, L, N, R) + cw or Cm.shape != Bm.shape:
        raise ValueError(f"Bm/Cm must be {(B, L, N, R) + cw}, got {Bm.shape} and {Cm.shape}")
    y = np.empty((B, L, D, R), dtype=np.float64)
    h_last = np.empty((B, D, N) + cw, dtype=np.float64)
    q_last = np.empty((B, D, N) + cw, dtype=np.float64)
    rc = lib.oracle_scan_mimo_f64(
        B, L, D, N, R, DISC[disc], int(bool(is_complex)),
        _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(theta), _ptr(lam),
        _ptr(h0), _ptr(q0), _ptr(y), _ptr(h_last), _ptr(q_last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_mimo_f64 returned {rc}")
    if return_q:
        return y, h_last, q_last
    return y, h_last


def combine(a2, b2, a1, b1):
    """(a2,b2)(x)(a1,b1) = (a2*a1, a2*b1 + b2) elementwise on complex arrays."""
    lib = _load()
    a2, b2, a1, b1 = (np.ascontiguousarray(np.asarray(v, dtype=np.complex128)) for v in (a2, b2, a1, b1))
    n = a2.size
    ao = np.empty(n, dtype=np.complex128)
    bo = np.empty(n, dtype=np.complex128)
    lib.oracle_combine_f64(n, *(x.ctypes.data_as(ctypes.c_void_p) for x in (a2, b2, a1, b1, ao, bo)))
    return ao.reshape(a2.shape), bo.reshape(a2.shape)
