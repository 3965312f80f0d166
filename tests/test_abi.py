"""C-ABI contract of libssmscan.so, checked without a GPU.

Every call here is rejected by the library's host-side validation before any
HIP call, so nothing is launched.  Fake device pointers are plain aligned
integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_42_amd import scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "ssm_calibrate.h")]

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
P = 0x10000  # an aligned fake device address (never dereferenced)


def declared_functions():
    names = set()
    for h in HEADERS:
        names |= set(re.findall(r"\b(ssm_(?:scan|ssd|mimo|calibrate)_\w+)\s*\(", open(h).read()))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = scan._lib()
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_step", "ssm_scan_bwd", "ssm_scan_workspace_bytes",
            "ssm_scan_bwd_workspace_bytes", "ssm_ssd_fwd", "ssm_ssd_workspace_bytes", "ssm_mimo_fwd",
            "ssm_mimo_step", "ssm_mimo_workspace_bytes", "ssm_scan_status_string", "ssm_scan_abi_version",
            "ssm_scan_last_hip_error", "ssm_scan_fwd_noalloc", "ssm_calibrate_stream",
            "ssm_calibrate_device_math"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    header_version = int(re.search(r"#define SSM_SCAN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert scan.ssm_scan_abi_version() == header_version == scan.ABI_VERSION == 5
    for code, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                       (3, "workspace too small"), (4, "HIP runtime error"), (99, "unknown status")]:
        assert scan.ssm_scan_status_string(code) == text
    assert scan._lib().ssm_scan_last_hip_error() == 0


def call(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=0, y=P, h=0, ws=0, ws_bytes=0):
    lib = scan._lib()
    dp = None if desc is None else ctypes.byref(desc)
    args = [u, delta, A, B, C, D, theta, lam, y, h, ws]
    return lib.ssm_scan_fwd(dp, *[ctypes.c_void_p(a) if a else None for a in args], ws_bytes, None)


def desc(B=1, L=8, D=4, N=4, dtype="f32", disc="euler", cplx=False, algo="auto"):
    return scan.make_desc(B, L, D, N, {"f32": 0, "bf16": 1}[dtype], disc, cplx, algo)


def test_null_descriptor_and_bad_sizes():
    assert call(None) == INVALID
    for kw in [dict(B=0), dict(L=0), dict(D=0), dict(N=0), dict(L=-3)]:
        assert call(desc(**kw)) == INVALID, kw
    assert scan.ssm_scan_workspace_bytes(desc(L=0)) == 0


def test_overflowing_sizes_rejected():
    assert call(desc(B=1 << 20, L=1 << 20, D=1 << 20, N=16)) == INVALID


def test_unsupported_modes():
    assert call(desc(N=65)) == UNSUPPORTED
    assert call(desc(disc="zoh", cplx=True)) == UNSUPPORTED
    d = desc()
    d.io_dtype = 7
    assert call(d) == UNSUPPORTED
    d = desc()
    d.disc = 3
    assert call(d) == UNSUPPORTED
    d = desc()
    d.algo = 9
    assert call(d) == UNSUPPORTED
    d = desc()
    d.is_complex = 2
    assert call(d) == UNSUPPORTED


def test_sweep_rules():
    # the lane sweep takes N <= 16, needs no workspace, and AUTO picks it only
    # once there are enough waves of 4 channels: 1536 for a real state, 2048
    # for complex exp-Euler, 3072 for the complex trapezoid
    assert call(desc(N=17, algo="sweep")) == UNSUPPORTED
    assert scan.ssm_scan_workspace_bytes(desc(algo="sweep")) == 0
    wide = desc(B=8, L=2048, D=1536, N=16, dtype="f32", disc="zoh", algo="auto")
    assert scan.ssm_scan_workspace_bytes(wide) == 0                       # 3072 waves: the sweep
    assert scan.ssm_scan_algo(wide) == "sweep"
    assert scan.ssm_scan_algo(desc(N=17)) == "sequential"
    assert scan.ssm_scan_algo(desc(algo="chunked")) == "chunked"
    narrow = desc(B=1, L=2048, D=1536, N=16, dtype="f32", disc="zoh", algo="auto")
    assert scan.ssm_scan_workspace_bytes(narrow) > 0                      # 384 waves: the chunked kernel
    assert scan.ssm_scan_algo(narrow) == "chunked"
    assert scan.ssm_scan_algo(desc(B=1, L=2048, D=6144, N=16, dtype="f32", disc="zoh", algo="auto")) == "sweep"
    assert scan.ssm_scan_algo(desc(B=1, L=2048, D=6140, N=16, dtype="f32", disc="zoh", algo="auto")) == "chunked"
    cplx = dict(L=4096, N=16, dtype="f32", cplx=True, algo="auto")
    assert scan.ssm_scan_algo(desc(B=4, D=2048, disc="euler", **cplx)) == "sweep"        # 2048 waves
    assert scan.ssm_scan_algo(desc(B=3, D=2048, disc="euler", **cplx)) == "chunked"      # 1536 waves
    assert scan.ssm_scan_algo(desc(B=4, D=2560, disc="trap", **cplx)) == "chunked"       # 2560 waves
    assert scan.ssm_scan_algo(desc(B=6, D=2048, disc="trap", **cplx)) == "sweep"         # 3072 waves
    # a sequence of at most one chunked tile (96 steps) always takes the sweep
    assert scan.ssm_scan_algo(desc(B=1, L=96, D=4, N=4, algo="auto")) == "sweep"
    assert scan.ssm_scan_algo(desc(B=1, L=97, D=4, N=4, algo="auto")) == "chunked"
    # 32-bit per-block offsets: 34 * D * N * esize must stay below 2^31
    assert call(desc(B=1, L=4, D=1 << 20, N=16, dtype="f32", algo="sweep")) == UNSUPPORTED


def test_required_pointers():
    for k in ["u", "delta", "A", "B", "C", "y"]:
        assert call(desc(), **{k: 0}) == INVALID, k


def test_lambda_and_theta_rules():
    assert call(desc(disc="trap")) == INVALID                  # trapezoid without lambda
    assert call(desc(disc="euler"), lam=P) == INVALID           # lambda given but unused
    assert call(desc(disc="zoh"), lam=P) == INVALID
    assert call(desc(cplx=False), theta=P) == INVALID           # theta on the real path


def test_alignment():
    assert call(desc(dtype="f32"), u=P + 2) == INVALID
    assert call(desc(dtype="bf16"), u=P + 1) == INVALID
    assert call(desc(dtype="f32"), A=P + 2) == INVALID
    assert call(desc(dtype="f32"), D=P + 2) == INVALID
    assert call(desc(cplx=True), h=P + 4) == INVALID            # complex h_last needs 8 bytes


def test_workspace_rules():
    # the sequential kernel needs no workspace
    assert scan.ssm_scan_workspace_bytes(desc(algo="sequential")) == 0
    d = desc(B=1, L=1 << 16, D=64, N=16, dtype="bf16", disc="trap", cplx=True, algo="chunked")
    need = scan.ssm_scan_workspace_bytes(d)
    if need == 0:
        pytest.skip("chunked kernel needs no workspace for this shape")
    assert call(d, lam=P, theta=P, ws=0) == WS_SMALL
    assert call(d, lam=P, theta=P, ws=P, ws_bytes=need - 1) == WS_SMALL
    assert call(d, lam=P, theta=P, ws=P + 64, ws_bytes=need) == INVALID  # not 256-byte aligned


def call_ex(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=0, h0=0, q0=0, y=P, h=0, q_last=0, ws=0,
            ws_bytes=0):
    lib = scan._lib()
    args = [u, delta, A, B, C, D, theta, lam, h0, q0, y, h, q_last, ws]
    return lib.ssm_scan_fwd_ex(ctypes.byref(desc), *[ctypes.c_void_p(a) if a else None for a in args], ws_bytes,
                               None)


def call_step(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=0, u_prev=0, B_prev=0, h=P, y=P):
    lib = scan._lib()
    dp = None if desc is None else ctypes.byref(desc)
    args = [u, delta, A, B, C, D, theta, lam, u_prev, B_prev, h, y]
    return lib.ssm_scan_step(dp, *[ctypes.c_void_p(a) if a else None for a in args], None)


def test_continuation_argument_rules():
    # q0 / q_last belong to the trapezoid only
    assert call_ex(desc(disc="euler"), q0=P) == INVALID
    assert call_ex(desc(disc="zoh"), q_last=P) == INVALID
    # state pointers aligned to one state element
    assert call_ex(desc(cplx=True), h0=P + 4) == INVALID
    assert call_ex(desc(disc="trap", cplx=True), lam=P, q0=P + 4) == INVALID
    assert call_ex(desc(disc="trap"), lam=P, q_last=P + 2) == INVALID
    # the same pointer rules as the plain scan
    assert call_ex(desc(), u=0) == INVALID
    assert call_ex(desc(disc="trap")) == INVALID
    assert call_ex(desc(N=65)) == UNSUPPORTED


def test_step_argument_rules():
    assert call_step(None) == INVALID
    assert call_step(desc(L=2)) == INVALID                              # one step per call
    assert call_step(desc(L=1), h=0) == INVALID                         # state required
    assert call_step(desc(L=1, disc="trap")) == INVALID                 # trapezoid needs lambda
    assert call_step(desc(L=1, disc="trap"), lam=P, u_prev=P) == INVALID  # u_prev and B_prev together
    assert call_step(desc(L=1, disc="trap"), lam=P, B_prev=P) == INVALID
    assert call_step(desc(L=1, disc="euler"), u_prev=P, B_prev=P) == INVALID  # trapezoid only
    assert call_step(desc(L=1, cplx=True), h=P + 4) == INVALID
    assert call_step(desc(L=1, disc="trap"), lam=P, u_prev=P + 2, B_prev=P) == INVALID
    assert call_step(desc(L=1), u=P + 2) == INVALID
    assert call_step(desc(L=1, N=65)) == UNSUPPORTED
    assert call_step(desc(L=1, disc="zoh", cplx=True)) == UNSUPPORTED


def call_bwd(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=0, h0=0, dy=P, dh=0, du=P, ddelta=P, dA=P,
             dB=P, dC=P, dD=0, dtheta=0, dlam=0, dh0=0, ws=P, ws_bytes=1 << 40):
    lib = scan._lib()
    args = [u, delta, A, B, C, D, theta, lam, h0, dy, dh, du, ddelta, dA, dB, dC, dD, dtheta, dlam, dh0, ws]
    return lib.ssm_scan_bwd(ctypes.byref(desc), *[ctypes.c_void_p(a) if a else None for a in args], ws_bytes, None)


def test_backward_argument_rules():
    for k in ["u", "dy", "du", "ddelta", "dA", "dB", "dC"]:
        assert call_bwd(desc(), **{k: 0}) == INVALID, k
    assert call_bwd(desc(disc="trap"), lam=P) == INVALID               # trapezoid needs dlambda
    assert call_bwd(desc(disc="euler"), dlam=P) == INVALID             # dlambda only for the trapezoid
    assert call_bwd(desc(cplx=True), dtheta=P) == INVALID              # dtheta needs theta
    assert call_bwd(desc(cplx=True), theta=P, dh0=P + 4) == INVALID    # complex state gradient: 8 bytes
    assert call_bwd(desc(), du=P + 2) == INVALID
    assert call_bwd(desc(N=65)) == UNSUPPORTED
    d = desc(B=2, L=100, D=8, N=16, cplx=True)
    need = scan.ssm_scan_bwd_workspace_bytes(d)
    assert need == 13 * 2 * 8 * 16 * 8                                 # ceil(100/8) snapshots of the state
    assert call_bwd(d, ws=0) == WS_SMALL
    assert call_bwd(d, ws_bytes=need - 1) == WS_SMALL
    assert call_bwd(d, ws=P + 64, ws_bytes=need) == INVALID            # not 256-byte aligned
    # a narrow, long problem: 512 segments of snapshots (rounded up to 256 bytes) plus 16
    # chunks of 256 steps (whole segments), one (Q, R) adjoint pair each per (b, d, n)
    r256 = lambda v: (v + 255) // 256 * 256
    d = desc(B=1, L=4096, D=8, N=16, cplx=True)
    assert scan.ssm_scan_bwd_workspace_bytes(d) == r256(512 * 8 * 16 * 8) + 16 * 8 * 16 * 16
    d = desc(B=1, L=4096, D=8, N=16)
    assert scan.ssm_scan_bwd_workspace_bytes(d) == r256(512 * 8 * 16 * 4) + 16 * 8 * 16 * 8


def call_ssd(desc, u=P, delta=P, A=P, B=P, C=P, D=0, y=P, h=0, ws=P, ws_bytes=1 << 40):
    lib = scan._lib()
    dp = None if desc is None else ctypes.byref(desc)
    args = [u, delta, A, B, C, D, y, h, ws]
    return lib.ssm_ssd_fwd(dp, *[ctypes.c_void_p(a) if a else None for a in args], ws_bytes, None)


def ssd_desc(B=1, L=100, D=128, N=16, P=64, dtype="bf16"):
    return scan.make_ssd_desc(B, L, D, N, P, {"f32": 0, "bf16": 1}[dtype])


def test_ssd_argument_rules():
    assert call_ssd(None) == INVALID
    for kw in [dict(B=0), dict(L=0), dict(D=0), dict(N=0), dict(P=0)]:
        assert call_ssd(ssd_desc(**kw)) == INVALID, kw
    assert call_ssd(ssd_desc(dtype="f32")) == UNSUPPORTED
    assert call_ssd(ssd_desc(P=32, D=128)) == UNSUPPORTED
    assert call_ssd(ssd_desc(D=100)) == UNSUPPORTED
    assert call_ssd(ssd_desc(N=65)) == UNSUPPORTED
    for k in ["u", "delta", "A", "B", "C", "y"]:
        assert call_ssd(ssd_desc(), **{k: 0}) == INVALID, k
    assert call_ssd(ssd_desc(), u=P + 1) == INVALID
    assert call_ssd(ssd_desc(), u=P + 8) == INVALID                      # u and y move in 16-byte rows
    assert call_ssd(ssd_desc(), y=P + 8) == INVALID
    d = ssd_desc(B=2, L=100, D=128, N=16)
    need = scan.ssm_ssd_workspace_bytes(d)
    assert need == 2 * (2 * 2 * 2 * 16 * 64 * 2) + 256           # 2 rows x 2 heads x 2 chunks, bf16 states
    assert call_ssd(d, ws=0) == WS_SMALL
    assert call_ssd(d, ws_bytes=need - 1) == WS_SMALL
    assert call_ssd(d, ws=P + 64, ws_bytes=need) == INVALID


def mimo_desc(B=1, L=8, D=4, N=4, R=4, dtype="bf16", disc="trap", cplx=True, chunk=0):
    return scan.make_mimo_desc(B, L, D, N, R, {"f32": 0, "bf16": 1}[dtype], disc, cplx, chunk)


def call_mimo(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=P, h0=0, q0=0, y=P, h=0, q=0, ws=0,
              ws_bytes=0):
    lib = scan._lib()
    dp = None if desc is None else ctypes.byref(desc)
    args = [u, delta, A, B, C, D, theta, lam, h0, q0, y, h, q, ws]
    return lib.ssm_mimo_fwd(dp, *[ctypes.c_void_p(a) if a else None for a in args], ws_bytes, None)


def call_mimo_step(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=P, u_prev=0, B_prev=0, h=P, y=P):
    lib = scan._lib()
    args = [u, delta, A, B, C, D, theta, lam, u_prev, B_prev, h, y]
    return lib.ssm_mimo_step(ctypes.byref(desc), *[ctypes.c_void_p(a) if a else None for a in args], None)


def test_mimo_descriptor_rules():
    assert call_mimo(None) == INVALID
    for kw in [dict(B=0), dict(L=0), dict(D=0), dict(N=0), dict(R=0), dict(chunk=-1)]:
        assert call_mimo(mimo_desc(**kw)) == INVALID, kw
    for kw in [dict(R=3), dict(R=16), dict(N=65)]:
        assert call_mimo(mimo_desc(**kw)) == UNSUPPORTED, kw
    assert call_mimo(mimo_desc(disc="zoh", cplx=True), lam=0) == UNSUPPORTED
    d = mimo_desc()
    d.reserved = 1
    assert call_mimo(d) == INVALID
    assert call_mimo(mimo_desc(B=1 << 20, L=1 << 20, D=1 << 20, N=16)) == INVALID
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(R=3)) == 0


def test_mimo_pointer_rules():
    assert call_mimo(mimo_desc(), u=0) == INVALID
    assert call_mimo(mimo_desc(), lam=0) == INVALID                       # the trapezoid needs lambda
    assert call_mimo(mimo_desc(disc="euler"), lam=P) == INVALID           # and only it takes one
    assert call_mimo(mimo_desc(disc="euler", cplx=False), lam=0, theta=P) == INVALID
    assert call_mimo(mimo_desc(disc="euler"), lam=0, q0=P) == INVALID     # q0, q_last: trapezoid only
    # u and y move in runs of R elements (here 8 bytes), B and C in runs of R complex elements (16 bytes)
    assert call_mimo(mimo_desc(), u=P + 4) == INVALID
    assert call_mimo(mimo_desc(), y=P + 4) == INVALID
    assert call_mimo(mimo_desc(), B=P + 8) == INVALID
    assert call_mimo(mimo_desc(), C=P + 8) == INVALID
    assert call_mimo(mimo_desc(), h0=P + 4) == INVALID                    # complex state: 8-byte elements


def test_mimo_workspace_follows_the_chunking():
    # one chunk (a wide problem, or a fixed chunk covering L): no workspace
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=64, D=4096, L=1000, N=16)) == 0
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(L=100, chunk=100)) == 0
    # a fixed chunk of 16 steps over 100: 7 chunks, 6 carried (P, h) pairs per (b, d, n)
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=2, D=3, N=5, L=100, chunk=16)) == 6 * 2 * 3 * 5 * 16
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=2, D=3, N=5, L=100, chunk=16, cplx=False)) == 6 * 2 * 3 * 5 * 8
    # the sequence is cut until there are 2^21 lanes, into chunks of at least 128 steps
    need = scan.ssm_mimo_workspace_bytes(mimo_desc(B=1, D=8, N=16, L=1 << 14))
    assert need == (128 - 1) * 8 * 16 * 16                               # 128 chunks of 128 steps
    # 2^16 lanes (8192 channels of 8 lanes): 32 chunks of 256 steps
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=4, D=2048, N=16, L=8192)) == 31 * 4 * 2048 * 16 * 16
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=2, D=2048, N=16, L=8192)) == 63 * 2 * 2048 * 16 * 16
    # 2^21 lanes: one chunk
    assert scan.ssm_mimo_workspace_bytes(mimo_desc(B=64, D=4096, N=16, L=8192)) == 0
    d = mimo_desc(L=100, chunk=16)
    assert call_mimo(d, ws=P, ws_bytes=scan.ssm_mimo_workspace_bytes(d) - 1) == WS_SMALL
    assert call_mimo(d, ws=0, ws_bytes=0) == WS_SMALL


def test_mimo_step_rules():
    assert call_mimo_step(mimo_desc(L=2)) == INVALID                      # one step
    assert call_mimo_step(mimo_desc(L=1), h=0) == INVALID
    assert call_mimo_step(mimo_desc(L=1), u_prev=P) == INVALID            # u_prev and B_prev together
    assert call_mimo_step(mimo_desc(L=1, disc="euler"), lam=0, u_prev=P, B_prev=P) == INVALID
    assert call_mimo_step(mimo_desc(L=1), u_prev=P + 4, B_prev=P) == INVALID
    assert call_mimo_step(mimo_desc(L=1, R=3)) == UNSUPPORTED


SCRATCH_LIMIT = 5
NOALLOC_BYTES = 64 << 20


def call_noalloc(desc, u=P, delta=P, A=P, B=P, C=P, D=0, theta=0, lam=0, y=P, h=0):
    lib = scan._lib()
    dp = None if desc is None else ctypes.byref(desc)
    args = [u, delta, A, B, C, D, theta, lam, y, h]
    return lib.ssm_scan_fwd_noalloc(dp, *[ctypes.c_void_p(a) if a else None for a in args], None)


def test_noalloc_limit_in_header():
    text = open(HEADER).read()
    assert "#define SSM_SCAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert "SSM_ERR_SCRATCH_LIMIT = 5" in text
    assert "scratch" in scan.ssm_scan_status_string(SCRATCH_LIMIT)


def test_noalloc_validates_before_any_hip_call():
    assert call_noalloc(None) == INVALID
    assert call_noalloc(desc(L=0)) == INVALID
    for k in ["u", "delta", "A", "B", "C", "y"]:
        assert call_noalloc(desc(), **{k: 0}) == INVALID, k
    assert call_noalloc(desc(disc="trap")) == INVALID             # no lambda
    assert call_noalloc(desc(N=65)) == UNSUPPORTED
    assert call_noalloc(desc(cplx=True), h=P + 4) == INVALID      # misaligned complex h_last


def test_noalloc_rejects_problems_beyond_its_scratch():
    big = desc(B=1, L=1 << 20, D=1024, N=16, dtype="bf16", disc="trap", cplx=True, algo="chunked")
    assert scan.ssm_scan_workspace_bytes(big) > NOALLOC_BYTES
    assert call_noalloc(big, lam=P, theta=P) == SCRATCH_LIMIT
    # the largest chunked problem that fits is accepted by the size check
    # (it would go on to look up the GPU's scratch, so it is not called here)
    small = desc(B=1, L=4096, D=64, N=16, dtype="bf16", disc="trap", cplx=True, algo="chunked")
    assert 0 < scan.ssm_scan_workspace_bytes(small) <= NOALLOC_BYTES


def test_calibrate_stream_argument_checks():
    lib = scan._lib()
    v = ctypes.c_void_p
    assert lib.ssm_calibrate_stream(None, 1 << 20, v(P), 1 << 16, 0, None, None) == INVALID
    assert lib.ssm_calibrate_stream(v(P), 1 << 20, None, 1 << 16, 0, None, None) == INVALID
    assert lib.ssm_calibrate_stream(v(P), 1000, v(P + (1 << 24)), 16, 0, None, None) == INVALID      # not a multiple
    assert lib.ssm_calibrate_stream(v(P), 65 * 16, v(P + (1 << 24)), 16, 0, None, None) == INVALID   # ratio above 64
    assert lib.ssm_calibrate_stream(v(P + 8), 320, v(P + (1 << 24)), 16, 0, None, None) == INVALID   # misaligned
    assert lib.ssm_calibrate_stream(v(P), 320, v(P + 16), 16, 0, None, None) == INVALID              # overlapping
    assert lib.ssm_calibrate_stream(v(P), 320, v(P + (1 << 24)), 16, 2, None, None) == INVALID       # bad flag
    assert lib.ssm_calibrate_stream(v(P), 320, v(P + (1 << 24)), 16, 0, v(P + 4), None) == INVALID   # clocks


def test_device_math_argument_checks():
    lib = scan._lib()
    v = ctypes.c_void_p
    X, Y, O = P, P + (1 << 20), P + (2 << 20)
    assert lib.ssm_calibrate_device_math(9, v(X), v(Y), v(O), 16, None) == INVALID    # unknown function
    assert lib.ssm_calibrate_device_math(-1, v(X), v(Y), v(O), 16, None) == INVALID
    assert lib.ssm_calibrate_device_math(0, v(X), None, v(O), 16, None) == INVALID    # exp needs y
    assert lib.ssm_calibrate_device_math(7, v(X), None, v(O), 16, None) == INVALID    # so does expm1
    assert lib.ssm_calibrate_device_math(1, None, None, v(O), 16, None) == INVALID
    assert lib.ssm_calibrate_device_math(1, v(X), None, None, 16, None) == INVALID
    assert lib.ssm_calibrate_device_math(1, v(X), None, v(X + 32), 16, None) == INVALID   # out overlaps x
    assert lib.ssm_calibrate_device_math(0, v(X), v(Y), v(Y + 32), 16, None) == INVALID   # out overlaps y
    assert lib.ssm_calibrate_device_math(1, v(X), None, v(O), -1, None) == INVALID
    assert lib.ssm_calibrate_device_math(1, v(X), None, v(O), 1 << 31, None) == INVALID
    assert lib.ssm_calibrate_device_math(1, v(X), None, v(O), 0, None) == 0               # nothing to do
