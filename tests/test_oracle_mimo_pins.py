"""Pins of the MIMO oracle (oracle.scan_mimo), independent of its own code.

The MIMO scan keeps one state per (b, d) and feeds it R inputs through the
columns of an N x R matrix B, reading R outputs through the columns of C
(ai.tomabc.com Mamba-3 story, MIMO section).  Three facts fix it:

* R = 1 is the single-input scan, itself pinned by test_oracle_pins.py:
  bit-identical results.
* Superposition: for fixed decays the state is linear in the input terms
  (and in h0, q0), so output r of the MIMO scan equals the sum over input
  columns r' of single-input scans fed (u[..., r'], B[..., r']) and read
  through C[..., r], plus D u[..., r].  A transposed B or C, a wrong column,
  a skip term counted per input, or a trapezoid that keeps only one column
  of the previous input fails this by O(1).
* With A = 0 and no rotation the decays are 1, and the state is a cumulative
  sum that numpy computes directly (exp-Euler and the trapezoid at
  lambda = 1/2).
A split run continued from (h_last, q_last) must equal the whole run bit for
bit.
"""
import numpy as np
import pytest

import oracle

MODES = [("zoh", False), ("euler", False), ("trap", False), ("euler", True), ("trap", True)]


def _problem(disc, cplx, seed, B=2, L=9, D=3, N=4, R=3, with_state=True):
    rng = np.random.default_rng(seed)
    cw = (2,) if cplx else ()
    return dict(
        u=rng.standard_normal((B, L, D, R)),
        delta=rng.uniform(0.05, 0.6, (B, L, D)),
        A=-rng.uniform(0.1, 2.0, (D, N)),
        Bm=rng.standard_normal((B, L, N, R) + cw),
        Cm=rng.standard_normal((B, L, N, R) + cw),
        Dskip=rng.standard_normal((D,)),
        theta=rng.uniform(-3.0, 3.0, (B, L, D, N)) if cplx else None,
        lam=rng.uniform(0.0, 1.0, (B, L, D)) if disc == "trap" else None,
        h0=rng.standard_normal((B, D, N) + cw) if with_state else None,
        q0=rng.standard_normal((B, D, N) + cw) if with_state and disc == "trap" else None,
    )


def _mimo(x, disc, cplx):
    return oracle.scan_mimo(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], x["Dskip"], x["theta"], x["lam"],
                            disc=disc, is_complex=cplx, h0=x["h0"], q0=x["q0"], nthreads=2, return_q=True)


@pytest.mark.parametrize("disc,cplx", MODES)
def test_rank_one_is_the_single_input_scan(disc, cplx):
    x = _problem(disc, cplx, seed=1, R=1)
    y, h, q = _mimo(x, disc, cplx)
    y1, h1, q1 = oracle.scan(x["u"][..., 0], x["delta"], x["A"], x["Bm"][:, :, :, 0], x["Cm"][:, :, :, 0],
                             x["Dskip"], x["theta"], x["lam"], disc=disc, is_complex=cplx, h0=x["h0"],
                             q0=x["q0"], nthreads=2, return_q=True)
    assert np.array_equal(y[..., 0], y1)
    assert np.array_equal(h, h1)
    if disc == "trap":
        assert np.array_equal(q, q1)


@pytest.mark.parametrize("disc,cplx", MODES)
def test_superposition_over_input_columns(disc, cplx):
    x = _problem(disc, cplx, seed=2)
    y, h, q = _mimo(x, disc, cplx)
    R = x["u"].shape[-1]
    y_sum = np.zeros_like(y)
    h_sum = np.zeros_like(h)
    q_sum = np.zeros_like(q)
    for rp in range(R):  # input column r'
        for r in range(R):  # output column r
            yr, hr, qr = oracle.scan(x["u"][..., rp], x["delta"], x["A"], x["Bm"][:, :, :, rp],
                                     x["Cm"][:, :, :, r], None, x["theta"], x["lam"], disc=disc, is_complex=cplx,
                                     h0=x["h0"] if rp == 0 else None, q0=x["q0"] if rp == 0 else None,
                                     nthreads=2, return_q=True)
            y_sum[..., r] += yr
        h_sum += hr
        q_sum += qr
    y_sum += x["Dskip"][None, None, :, None] * x["u"]
    scale = np.max(np.abs(y))
    assert np.max(np.abs(y - y_sum)) <= 1e-12 * scale
    assert np.max(np.abs(h - h_sum)) <= 1e-12 * np.max(np.abs(h))
    if disc == "trap":
        assert np.max(np.abs(q - q_sum)) <= 1e-12 * np.max(np.abs(q))


@pytest.mark.parametrize("disc", ["euler", "trap"])
@pytest.mark.parametrize("cplx", [False, True])
def test_unit_decay_is_a_cumulative_sum(disc, cplx):
    """A = 0, theta = 0, constant delta, B and C: alpha = 1, so
    exp-Euler:        h_t = delta sum_r B[:, r] cumsum(u_r)_t
    trapezoid (1/2):  h_t = delta sum_r B[:, r] (cumsum(u_r)_t - u_{r,t} / 2)."""
    rng = np.random.default_rng(3)
    Bn, L, D, N, R = 1, 12, 2, 3, 4
    dt = 0.3
    u = rng.standard_normal((Bn, L, D, R))
    Bc = rng.standard_normal((N, R)) + (1j * rng.standard_normal((N, R)) if cplx else 0)
    Cc = rng.standard_normal((N, R)) + (1j * rng.standard_normal((N, R)) if cplx else 0)
    Dskip = rng.standard_normal(D)

    def stored(M):
        full = np.broadcast_to(M, (Bn, L, N, R))
        return np.stack([full.real, full.imag], axis=-1) if cplx else full.real.copy()

    lam = np.full((Bn, L, D), 0.5) if disc == "trap" else None
    y, h = oracle.scan_mimo(u, np.full((Bn, L, D), dt), np.zeros((D, N)), stored(Bc), stored(Cc), Dskip,
                            None, lam, disc=disc, is_complex=cplx)
    cs = np.cumsum(u, axis=1)
    if disc == "trap":
        cs = cs - u / 2
    # state (b, t, d, n) = dt * sum_r B[n, r] cs[b, t, d, r]
    state = dt * np.einsum("nr,btdr->btdn", Bc, cs)
    y_ref = np.einsum("nr,btdn->btdr", Cc, state).real + Dskip[None, None, :, None] * u
    assert np.max(np.abs(y - y_ref)) <= 1e-12 * np.max(np.abs(y_ref))
    h_ref = state[:, -1]
    h_c = h[..., 0] + 1j * h[..., 1] if cplx else h
    assert np.max(np.abs(h_c - h_ref)) <= 1e-12 * np.max(np.abs(h_ref))


@pytest.mark.parametrize("disc,cplx", [("trap", True), ("zoh", False)])
def test_split_run_continues_exactly(disc, cplx):
    x = _problem(disc, cplx, seed=4, L=11, with_state=False)
    y, h, q = _mimo(x, disc, cplx)
    L1 = 5
    first = {k: (v[:, :L1] if k in ("u", "delta", "Bm", "Cm", "theta", "lam") and v is not None else v)
             for k, v in x.items()}
    second = {k: (v[:, L1:] if k in ("u", "delta", "Bm", "Cm", "theta", "lam") and v is not None else v)
              for k, v in x.items()}
    ya, ha, qa = _mimo(first, disc, cplx)
    second["h0"], second["q0"] = ha, (qa if disc == "trap" else None)
    yb, hb, qb = _mimo(second, disc, cplx)
    assert np.array_equal(np.concatenate([ya, yb], axis=1), y)
    assert np.array_equal(hb, h)


def test_invalid_arguments_are_rejected():
    x = _problem("euler", True, seed=5)
    with pytest.raises(ValueError):
        oracle.scan_mimo(x["u"], x["delta"], x["A"], x["Bm"][:, :, :2], x["Cm"], disc="euler", is_complex=True)
    with pytest.raises(ValueError):  # complex ZOH is not defined
        oracle.scan_mimo(x["u"], x["delta"], x["A"], x["Bm"], x["Cm"], disc="zoh", is_complex=True)
