"""The kernel-argument layout the parameter re-read relies on (CPU only).

The scan kernel and the backward's reverse-sweep kernel read their parameter
structs back from the kernel-argument segment at a fixed offset: the first
struct at offset 0 and, for the scan kernel, the layout struct right after
the parameter struct at its natural alignment.  This compiles a probe kernel
with the same argument list for gfx950 and checks those offsets in the code
object's argument metadata, so a toolchain or struct change that moves them
fails here instead of on a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_42_amd", "csrc")

PROBE = r"""
#include "kernel_chunked.h"
#include "kernel_backward.h"
__global__ void probe_scan(ssm::ChunkParams p, ssm::ChunkLayout l) {}
__global__ void probe_bwd(ssm::BwdParams p) {}
"""


def _kernel_args(asm: str, kernel: str):
    """(offset, size) of each explicit argument of `kernel` in the metadata."""
    blocks = asm.split("  - .agpr_count:")
    for blk in blocks:
        if f".name:           {kernel}" in blk or re.search(rf"\.name:\s+{kernel}\b", blk):
            args = re.findall(r"- \.offset:\s+(\d+)\s+\.size:\s+(\d+)\s+\.value_kind:\s+by_value", blk)
            return [(int(o), int(s)) for o, s in args]
    raise AssertionError(f"no metadata for {kernel}")


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_parameter_structs_at_the_offsets_the_kernels_read(tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    out = tmp_path / "probe.s"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17", "--cuda-device-only", "-S",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(out), str(src)],
                   check=True, capture_output=True)
    asm = out.read_text()
    scan = _kernel_args(asm, "_Z10probe_scanN3ssm11ChunkParamsENS_11ChunkLayoutE")
    assert len(scan) == 2 and scan[0][0] == 0
    (off0, size0), (off1, _) = scan
    # the layout struct holds 64-bit fields: 8-byte alignment after the parameters
    assert off1 == (size0 + 7) // 8 * 8, scan
    bwd = _kernel_args(asm, "_Z9probe_bwdN3ssm9BwdParamsE")
    assert len(bwd) == 1 and bwd[0][0] == 0
