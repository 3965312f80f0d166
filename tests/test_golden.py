"""The oracle still reproduces the stored fixtures in tests/golden (CPU)."""
import glob
import os

import numpy as np
import pytest

import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.npz")))


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_oracle_reproduces_fixture(path):
    z = np.load(path)
    disc, cplx, _ = (str(v) for v in z["meta"])
    get = lambda k: z[k] if k in z.files else None  # noqa: E731
    y, h = oracle.scan(z["u"], z["delta"], z["A"], z["Bm"], z["Cm"], get("Dskip"), get("theta"), get("lam"),
                       disc=disc, is_complex=cplx == "1", nthreads=2)
    assert np.array_equal(y, z["y"])
    assert np.array_equal(h, z["h_last"])
