"""Pins of the oracle's gradients (oracle.scan_bwd) against finite differences.

The reverse sweep in oracle/ssm_oracle_bwd.c is checked against central
finite differences of the forward oracle, which is itself pinned to closed
forms and special cases (test_oracle_pins.py).  For
    L = sum(dy * y) + <dh_last, h_last>
every element of every input is perturbed by +-eps and
(L(x + eps) - L(x - eps)) / (2 eps) is compared with the analytic gradient.
In fp64 with eps ~ 1e-6 the difference quotient is good to ~1e-9 relative,
so a dropped term, a wrong sign or a missing conjugate (all O(1) errors)
fails by many orders of magnitude.  Every discretisation and both state
kinds are covered, with a nonzero initial state, and ZOH with A = 0 and a
tiny A (its limit and series branches).
"""
import numpy as np
import pytest

import oracle

MODES = [("zoh", False), ("euler", False), ("trap", False), ("euler", True), ("trap", True)]
REL = 1e-6


def _problem(disc, cplx, seed, B=2, L=6, D=2, N=3, big_theta=False):
    rng = np.random.default_rng(seed)
    cw = (2,) if cplx else ()
    x = dict(
        u=rng.standard_normal((B, L, D)),
        delta=rng.uniform(0.05, 0.6, (B, L, D)),
        A=-rng.uniform(0.1, 2.0, (D, N)),
        Bm=rng.standard_normal((B, L, N) + cw),
        Cm=rng.standard_normal((B, L, N) + cw),
        Dskip=rng.standard_normal((D,)),
        theta=rng.uniform(-3.0, 3.0, (B, L, D, N)) * (10.0 if big_theta else 1.0) if cplx else None,
        lam=rng.uniform(0.0, 1.0, (B, L, D)) if disc == "trap" else None,
        h0=rng.standard_normal((B, D, N) + cw),
    )
    if disc == "zoh":  # the A = 0 limit and the small-z series branch
        x["A"][0, 0] = 0.0
        x["A"][1, 1] = -1e-7
    dy = rng.standard_normal((B, L, D))
    dh = rng.standard_normal((B, D, N) + cw)
    return x, dy, dh


def _loss(x, disc, cplx, dy, dh):
    y, h = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                       disc=disc, is_complex=cplx, h0=x["h0"], nthreads=1)
    return float(np.sum(dy * y) + np.sum(dh * h))


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "Dskip": "dD", "theta": "dtheta",
           "lam": "dlambda", "h0": "dh0"}


def _check_all(disc, cplx, seed, **kw):
    x, dy, dh = _problem(disc, cplx, seed, **kw)
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                        disc=disc, is_complex=cplx, dy=dy, dh_last=dh, h0=x["h0"])
    worst = {}
    for name, gname in GRAD_OF.items():
        if x[name] is None:
            assert g[gname] is None
            continue
        an = g[gname]
        assert an.shape == x[name].shape, name
        fd = np.empty_like(an)
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            eps = 1e-6 * max(1.0, abs(v))
            flat[i] = v + eps
            lp = _loss(x, disc, cplx, dy, dh)
            flat[i] = v - eps
            lm = _loss(x, disc, cplx, dy, dh)
            flat[i] = v
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        scale = max(float(np.max(np.abs(fd))), 1e-12)
        worst[name] = float(np.max(np.abs(fd - an))) / scale
    return worst


@pytest.mark.parametrize("disc,cplx", MODES)
def test_gradients_match_finite_differences(disc, cplx):
    worst = _check_all(disc, cplx, seed=3)
    assert max(worst.values()) < REL, worst


def test_complex_gradients_with_wide_angles():
    """Rotation angles up to 30 rad (many turns per step)."""
    worst = _check_all("trap", True, seed=4, big_theta=True)
    assert max(worst.values()) < REL, worst


def test_gradient_of_linear_output_is_the_adjoint():
    """With everything but u fixed, y is linear in u, so <dy, J du> = <du_grad, du>
    for any direction du (a second, exact check of du on a longer sequence)."""
    disc, cplx = "trap", True
    x, dy, _ = _problem(disc, cplx, seed=5, B=1, L=40, D=3, N=4)
    x["h0"] = None
    y0, _ = oracle.scan(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                        disc=disc, is_complex=cplx)
    rng = np.random.default_rng(6)
    v = rng.standard_normal(x["u"].shape)
    y1, _ = oracle.scan(x["u"] + v, x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                        disc=disc, is_complex=cplx)
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                        disc=disc, is_complex=cplx, dy=dy)
    lhs = float(np.sum(dy * (y1 - y0)))
    rhs = float(np.sum(g["du"] * v))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)), (lhs, rhs)


def test_zero_upstream_gives_zero_gradients():
    x, dy, dh = _problem("trap", True, seed=7)
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                        disc="trap", is_complex=True, dy=np.zeros_like(dy), dh_last=np.zeros_like(dh), h0=x["h0"])
    for k, v in g.items():
        if v is not None:
            assert np.all(v == 0.0), k
