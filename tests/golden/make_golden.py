"""Write tests/golden/*.npz: seeded small inputs and the fp64 oracle's outputs.

Calls only the input generator and oracle/ (never the HIP path).  The pages
print no numeric worked example, so these fixtures are regression anchors for
the oracle and ready-made parity cases for the GPU tests, not page values.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from selective_state_space_42_amd.inputs import WORKLOADS, all_channels, make_inputs  # noqa: E402

CASES = {
    # the small real ZOH workload at its full size
    "real_zoh_b1_d4_l64_n4": WORKLOADS["real_zoh_b1_d4_l64_n4"],
    # a small complex exp-trapezoidal bf16 case with a ragged length
    "complex_trap_bf16_b2_d5_l77_n16": WORKLOADS["complex_trap_bf16_b4_d2560_l8192_n16"].scaled(
        name="complex_trap_bf16_b2_d5_l77_n16", batch=2, dim=5, seqlen=77),
}


def main():
    for name, w in CASES.items():
        t = make_inputs(w, seed=7, device="cpu")
        x = all_channels(t)
        y, h = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                           disc=w.disc, is_complex=w.is_complex, nthreads=1)
        arrays = {k: v for k, v in x.items() if v is not None}
        np.savez_compressed(os.path.join(HERE, f"{name}.npz"), y=y, h_last=h, **arrays,
                            meta=np.array([w.disc, str(int(w.is_complex)), w.io_dtype]))
        print(name, y.shape, float(np.abs(y).max()))


if __name__ == "__main__":
    main()
