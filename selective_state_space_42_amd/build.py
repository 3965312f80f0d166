"""Build libssmscan.so (HIP, gfx950) in-tree with hipcc.

    python -m selective_state_space_42_amd.build

Every HIP source is compiled with packed-fp32 instruction selection turned
off (-target-feature -packed-fp32-ops): scalar fp32 arithmetic only.  The
atomic optimizer is off too: it rewrites a single lane's ticket fetch-add into
a wave-wide form that consumes the returned value at once, so the wave would
wait a full memory round trip for a ticket it only needs a tile later.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssmscan.so")
# the same library with the look-back test delays compiled in (tests only: the
# ordering test of the chunked kernel's decoupled look-back loads it)
LOOKBACK_TEST_LIB = os.path.join(PKG, "libssmscan_lookback_test.so")
LOOKBACK_TEST_DELAY = 12
SOURCES = [os.path.join(CSRC, "ssm_scan.hip"), os.path.join(CSRC, "mimo.hip"), os.path.join(CSRC, "calibrate.hip")]
HEADERS = [os.path.join(ROOT, "include", "ssm_scan.h"), os.path.join(ROOT, "include", "ssm_calibrate.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]
ARCH = os.environ.get("SSM_OFFLOAD_ARCH", "gfx950")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc_cmd(out: str = LIB, extra=()):
    """One hipcc line that compiles and links every source (for inspection)."""
    return ["hipcc", *FLAGS, "-shared", *extra, "-o", out, *SOURCES]


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed linking {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the sources to objects in parallel, then link the library and
    its look-back test variant (the chunked kernel's translation unit compiled
    again with the test delays, linked with the same other objects)."""
    import tempfile

    with tempfile.TemporaryDirectory(prefix="ssmscan_build_") as tmpdir:
        jobs = [(src, os.path.join(tmpdir, os.path.basename(src) + ".o"), []) for src in SOURCES]
        test_obj = os.path.join(tmpdir, "lookback_test_" + os.path.basename(SOURCES[0]) + ".o")
        jobs.append((SOURCES[0], test_obj, [f"-DSSM_LOOKBACK_TEST_DELAY={LOOKBACK_TEST_DELAY}"]))
        procs = []
        for src, obj, extra in jobs:
            cmd = ["hipcc", *FLAGS, *extra, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd))
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src))
        failed = False
        for proc, src in procs:
            out, _ = proc.communicate()
            if proc.returncode != 0:
                sys.stderr.write(out)
                failed = True
        if failed:
            raise RuntimeError("hipcc failed building libssmscan.so")
        objs = [obj for _, obj, _ in jobs[:len(SOURCES)]]
        _link(objs, LIB, verbose)
        _link([test_obj] + objs[1:], LOOKBACK_TEST_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
