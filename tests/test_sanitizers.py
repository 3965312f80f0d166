"""Host-side sanitizer runs (CPU only, no GPU needed).

* The fp64 oracle (oracle/*.c) built by gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer runs its pin tests and the golden fixtures.
* The library's host code -- descriptor and pointer validation, the 64-bit
  size arithmetic, workspace layouts, the no-allocation entry point's limits --
  built by hipcc with both sanitizers on the host side only (device code is
  compiled as usual and never runs here) runs the C ABI and binding tests.

Each run is a subprocess with the matching sanitizer runtime preloaded and
leak detection off (the Python interpreter keeps its allocations).  Every
sanitizer report aborts that process (-fno-sanitize-recover=all), which fails
the test.  The builds go to a temporary directory; nothing here touches the
in-tree libraries.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_42_amd", "csrc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run_pytest(files, env_extra, timeout):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
    return r.stdout


def _have(tool):
    return subprocess.run(["which", tool], capture_output=True).returncode == 0


@pytest.mark.skipif(not _have("gcc"), reason="gcc not found")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "oracle", "*.c")))
    # the oracle's own flags (no fast-math, no FMA contraction) plus the sanitizers
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    "-pthread", *SAN, "-o", lib, *srcs, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    files = [os.path.join("tests", f) for f in ("test_oracle_pins.py", "test_oracle_bwd_pins.py",
                                                 "test_oracle_mimo_pins.py", "test_golden.py")]
    _run_pytest(files, {"SSM_ORACLE_LIB": lib, "LD_PRELOAD": asan}, timeout=600)


def _clang_asan_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.skipif(not _have("hipcc") or _clang_asan_runtime() is None, reason="hipcc or clang ASan runtime missing")
def test_host_validation_under_asan_ubsan(tmp_path):
    from selective_state_space_42_amd import build as B

    # the library's own flags with the sanitizers on the host side only
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    procs, objs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        procs.append(subprocess.Popen(["hipcc", *flags, *host_san, "-c", "-o", obj, src],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-3000:]
    lib = str(tmp_path / "libssmscan_san.so")
    subprocess.run(["hipcc", f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs], check=True, capture_output=True)
    files = [os.path.join("tests", f) for f in ("test_abi.py", "test_binding_checks.py")]
    _run_pytest(files, {"SSM_SCAN_LIB": lib, "LD_PRELOAD": _clang_asan_runtime()}, timeout=600)
