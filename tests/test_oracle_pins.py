"""Pins for the fp64 oracle: each test checks it against something other than itself.

Every expected value here comes from a closed form, a textbook special case,
a library routine (numpy cumsum / convolve) or an invariant -- never from the
oracle and never from the HIP path.  Sources of the definitions are the pages'
sections cited in oracle/ssm_oracle.c.  The pages print no numeric worked
example, so the worked values below are derived by hand from the definition
(the derivation is in each test's docstring).

CPU only (no GPU marker).
"""
import math

import numpy as np
import pytest

import oracle

MODES = [("zoh", False), ("euler", False), ("trap", False), ("euler", True), ("trap", True)]


def softplus(x):
    return np.log1p(np.exp(x))


def rand_problem(rng, B, L, D, N, disc, cplx, with_theta=True):
    u = rng.normal(size=(B, L, D))
    delta = softplus(rng.normal(-1.0, 0.5, size=(B, L, D)))
    A = -np.exp(rng.uniform(-2.0, 0.5, size=(D, N)))
    bc_shape = (B, L, N, 2) if cplx else (B, L, N)
    Bm = rng.normal(size=bc_shape)
    Cm = rng.normal(size=bc_shape)
    Dskip = rng.normal(size=D)
    theta = rng.uniform(-1.0, 1.0, size=(B, L, D, N)) if (cplx and with_theta) else None
    lam = 1.0 / (1.0 + np.exp(-rng.normal(size=(B, L, D)))) if disc == "trap" else None
    return dict(u=u, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, theta=theta, lam=lam)


def as_complex(x, cplx):
    return x[..., 0] + 1j * x[..., 1] if cplx else x.astype(np.complex128)


def run(p, disc, cplx, **kw):
    return oracle.scan(p["u"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dskip"], p["theta"], p["lam"],
                       disc=disc, is_complex=cplx, **kw)


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def discrete_terms(p, b, d, disc, cplx):
    """alpha_t[n], bterm_t[n] for one channel, vectorised over t (numpy, not the oracle)."""
    dt = p["delta"][b, :, d]
    A = p["A"][d]
    z = dt[:, None] * A[None, :]
    rot = np.exp(1j * p["theta"][b, :, d, :]) if (cplx and p["theta"] is not None) else 1.0
    alpha = np.exp(z) * rot
    q = as_complex(p["Bm"], cplx)[b] * p["u"][b, :, d][:, None]
    if disc == "zoh":
        with np.errstate(divide="ignore", invalid="ignore"):
            gamma = np.where(A[None, :] != 0, np.expm1(z) / A[None, :], dt[:, None])
        bterm = gamma * q
    elif disc == "euler":
        bterm = dt[:, None] * q
    else:
        lam = p["lam"][b, :, d][:, None]
        qprev = np.vstack([np.zeros((1, q.shape[1])), q[:-1]])
        bterm = lam * dt[:, None] * q + (1 - lam) * dt[:, None] * alpha * qprev
    return alpha, bterm


# ---------------------------------------------------------------- P-a
@pytest.mark.parametrize("disc,cplx", MODES)
def test_closed_form_sum_of_products(disc, cplx):
    """h_t = sum_{s<=t} (prod_{s<r<=t} alpha_r) b_s  (brute force, O(L^2 N)).

    The unrolled form of the recurrence in the operator derivation of the
    complex-parallel-scan page; y_t = Re sum_n C_t h_t + D u_t (post-update).
    """
    rng = np.random.default_rng(1)
    B, L, D, N = 2, 40, 3, 4
    p = rand_problem(rng, B, L, D, N, disc, cplx)
    y, h = run(p, disc, cplx)
    Cc = as_complex(p["Cm"], cplx)
    y_ref = np.empty_like(y)
    h_ref = np.empty((B, D, N), dtype=np.complex128)
    for b in range(B):
        for d in range(D):
            alpha, bterm = discrete_terms(p, b, d, disc, cplx)
            H = np.zeros((L, N), dtype=np.complex128)
            for t in range(L):
                P = np.ones((t + 1, N), dtype=np.complex128)
                for s in range(t - 1, -1, -1):
                    P[s] = P[s + 1] * alpha[s + 1]
                H[t] = (P * bterm[: t + 1]).sum(axis=0)
            y_ref[b, :, d] = (Cc[b] * H).sum(axis=1).real + p["Dskip"][d] * p["u"][b, :, d]
            h_ref[b, d] = H[-1]
    assert rel_err(y, y_ref) < 1e-12
    h_c = as_complex(h, cplx) if cplx else h
    assert rel_err(h_c, h_ref if cplx else h_ref.real) < 1e-12


# ---------------------------------------------------------------- P-b
def test_combine_associative_and_ordered():
    """(O3 O2) O1 = O3 (O2 O1), and O2 O1 applied to h equals O1 then O2."""
    rng = np.random.default_rng(2)
    n = 257
    ops = [(rng.normal(size=n) + 1j * rng.normal(size=n), rng.normal(size=n) + 1j * rng.normal(size=n))
           for _ in range(3)]
    (a1, b1), (a2, b2), (a3, b3) = ops
    a32, b32 = oracle.combine(a3, b3, a2, b2)
    left = oracle.combine(a32, b32, a1, b1)
    a21, b21 = oracle.combine(a2, b2, a1, b1)
    right = oracle.combine(a3, b3, a21, b21)
    for l, r in zip(left, right):
        assert rel_err(l, r) < 1e-14
    h = rng.normal(size=n) + 1j * rng.normal(size=n)
    seq = a2 * (a1 * h + b1) + b2
    assert rel_err(a21 * h + b21, seq) < 1e-14
    # a plausible mistake, the operands swapped, must not pass this check
    a12, b12 = oracle.combine(a1, b1, a2, b2)
    assert rel_err(a12 * h + b12, seq) > 1e-3


# ---------------------------------------------------------------- P-c
@pytest.mark.parametrize("disc", ["euler", "trap"])
def test_theta_zero_complex_reduces_to_real(disc):
    """theta = 0 and Im B = Im C = 0: the complex path equals the real path."""
    rng = np.random.default_rng(3)
    pr = rand_problem(rng, 2, 33, 3, 5, disc, False)
    pc = dict(pr)
    pc["Bm"] = np.stack([pr["Bm"], np.zeros_like(pr["Bm"])], axis=-1)
    pc["Cm"] = np.stack([pr["Cm"], np.zeros_like(pr["Cm"])], axis=-1)
    pc["theta"] = np.zeros(pr["u"].shape + (5,))
    yr, hr = run(pr, disc, False)
    yc, hc = run(pc, disc, True)
    assert rel_err(yc, yr) < 1e-15
    assert rel_err(hc[..., 0], hr) < 1e-15
    assert np.max(np.abs(hc[..., 1])) == 0.0
    # theta omitted (NULL) means theta = 0
    pc["theta"] = None
    yn, _ = run(pc, disc, True)
    assert rel_err(yn, yr) < 1e-15


@pytest.mark.parametrize("disc", ["euler", "trap"])
def test_theta_zero_complex_split_identity(disc):
    """With real alpha the scan is linear in B, so for complex B, C:
    y_c = y_r(B_re, C_re) - y_r(B_im, C_im) + D u   (both y_r with D = 0).
    A conjugated C, or a sign slip in Re(C h), fails this."""
    rng = np.random.default_rng(4)
    pc = rand_problem(rng, 1, 29, 2, 3, disc, True, with_theta=False)
    yc, _ = run(pc, disc, True)
    base = dict(pc, Dskip=None, theta=None)
    y1, _ = run(dict(base, Bm=pc["Bm"][..., 0], Cm=pc["Cm"][..., 0]), disc, False)
    y2, _ = run(dict(base, Bm=pc["Bm"][..., 1], Cm=pc["Cm"][..., 1]), disc, False)
    expect = y1 - y2 + pc["Dskip"][None, None, :] * pc["u"]
    assert rel_err(yc, expect) < 1e-13


# ---------------------------------------------------------------- P-d
@pytest.mark.parametrize("cplx", [False, True])
def test_trap_lambda_one_is_exp_euler(cplx):
    """lambda = 1 gives beta = 0 and gamma = delta: exactly exp-Euler
    (discretisation table of the Mamba-3 story page)."""
    rng = np.random.default_rng(5)
    p = rand_problem(rng, 2, 31, 3, 4, "trap", cplx)
    p["lam"] = np.ones_like(p["u"])
    yt, ht = run(p, "trap", cplx)
    ye, he = run(dict(p, lam=None), "euler", cplx)
    assert np.array_equal(yt, ye)
    assert np.array_equal(ht, he)


# ---------------------------------------------------------------- P-e
@pytest.mark.parametrize("cplx", [False, True])
def test_trap_two_band_closed_form(cplx):
    """Exp-trapezoidal as a two-band weighted sum (decay mask times a two-band
    mask, the L_decay o L_conv structure of the Mamba-3 story page):
      y_t = Re sum_n C_t sum_{s<=t} P(s,t) w(s,t) B_s u_s + D u_t
      P(s,t) = prod_{s<r<=t} alpha_r,  w(t,t) = lam_t d_t,
      w(s,t) = lam_s d_s + (1 - lam_{s+1}) d_{s+1}   for s < t.
    A beta term placed on the wrong step, or lambda and 1-lambda swapped,
    fails this."""
    rng = np.random.default_rng(6)
    B, L, D, N = 1, 37, 2, 3
    p = rand_problem(rng, B, L, D, N, "trap", cplx)
    y, _ = run(p, "trap", cplx)
    Bc = as_complex(p["Bm"], cplx)
    Cc = as_complex(p["Cm"], cplx)
    y_ref = np.empty_like(y)
    for d in range(D):
        alpha, _ = discrete_terms(p, 0, d, "trap", cplx)
        dt = p["delta"][0, :, d]
        lam = p["lam"][0, :, d]
        u = p["u"][0, :, d]
        for t in range(L):
            acc = np.zeros(N, dtype=np.complex128)
            Pst = np.ones(N, dtype=np.complex128)
            for s in range(t, -1, -1):
                if s < t:
                    Pst = Pst * alpha[s + 1]
                w = lam[s] * dt[s] if s == t else lam[s] * dt[s] + (1 - lam[s + 1]) * dt[s + 1]
                acc += Pst * w * Bc[0, s] * u[s]
            y_ref[0, t, d] = (Cc[0, t] * acc).sum().real + p["Dskip"][d] * u[t]
    assert rel_err(y, y_ref) < 1e-12


# ---------------------------------------------------------------- P-f
def test_special_cases_cumsum():
    """A = 0, theta = 0, constant delta and B (per n):
       exp-Euler:           h_t = delta B cumsum(u)_t
       exp-trap, lambda=1/2: h_t = delta B (cumsum(u)_t - u_t/2)
       ZOH with A = 0 takes the limit delta, i.e. equals exp-Euler; A -> 0 too."""
    rng = np.random.default_rng(7)
    L, N = 50, 3
    u = rng.normal(size=(1, L, 1))
    dlt = 0.37
    Bn = rng.normal(size=N)
    Cn = rng.normal(size=N)
    base = dict(u=u, delta=np.full((1, L, 1), dlt), A=np.zeros((1, N)),
                Bm=np.broadcast_to(Bn, (1, L, N)).copy(), Cm=np.broadcast_to(Cn, (1, L, N)).copy(),
                Dskip=None, theta=None, lam=None)
    cs = np.cumsum(u[0, :, 0])
    ye, he = run(base, "euler", False)
    assert rel_err(ye[0, :, 0], dlt * cs * (Cn * Bn).sum()) < 1e-12
    assert rel_err(he[0, 0], dlt * Bn * cs[-1]) < 1e-12
    yt, ht = run(dict(base, lam=np.full((1, L, 1), 0.5)), "trap", False)
    assert rel_err(yt[0, :, 0], dlt * (cs - u[0, :, 0] / 2) * (Cn * Bn).sum()) < 1e-12
    yz, _ = run(base, "zoh", False)
    assert rel_err(yz, ye) < 1e-15
    yz2, _ = run(dict(base, A=np.full((1, N), -1e-12)), "zoh", False)
    assert rel_err(yz2, ye) < 1e-9


@pytest.mark.parametrize("disc,cplx", MODES)
def test_special_case_lti_convolution(disc, cplx):
    """Constant delta, A, B, C, theta, lambda make the scan LTI: y = u * K + D u
    (causal convolution, numpy.convolve) with K_k = Re sum_n C alpha^k g_k B, where
    g_k = gamma for the ZOH and exp-Euler forms; for exp-trap K_0 uses lam*delta
    and K_k (k >= 1) uses delta (the two trapezoid weights add up)."""
    rng = np.random.default_rng(8)
    L, N = 64, 4
    u = rng.normal(size=(1, L, 1))
    dlt = 0.21
    A = -np.exp(rng.uniform(-1.5, 0.5, size=N))
    Bn = rng.normal(size=(N, 2)) if cplx else rng.normal(size=N)
    Cn = rng.normal(size=(N, 2)) if cplx else rng.normal(size=N)
    th = rng.uniform(-1, 1, size=N) if cplx else None
    lam = 0.3
    p = dict(u=u, delta=np.full((1, L, 1), dlt), A=A[None, :],
             Bm=np.broadcast_to(Bn, (1, L) + Bn.shape).copy(), Cm=np.broadcast_to(Cn, (1, L) + Cn.shape).copy(),
             Dskip=np.array([0.7]), theta=None if th is None else np.broadcast_to(th, (1, L, 1, N)).copy(),
             lam=np.full((1, L, 1), lam) if disc == "trap" else None)
    y, _ = run(p, disc, cplx)
    alpha = np.exp(dlt * A) * (np.exp(1j * th) if cplx else 1.0)
    Bc = as_complex(Bn, cplx)
    Cc = as_complex(Cn, cplx)
    k = np.arange(L)[:, None]
    if disc == "zoh":
        g = np.broadcast_to(np.expm1(dlt * A) / A, (L, N))
    elif disc == "euler":
        g = np.full((L, N), dlt)
    else:
        g = np.full((L, N), dlt)
        g[0] = lam * dlt
    K = (Cc[None, :] * alpha[None, :] ** k * g * Bc[None, :]).sum(axis=1).real
    y_ref = np.convolve(u[0, :, 0], K)[:L] + 0.7 * u[0, :, 0]
    assert rel_err(y[0, :, 0], y_ref) < 1e-12


# ---------------------------------------------------------------- P-g
LN2 = math.log(2.0)


def _scalar_case(disc, lam=None, L=24):
    p = dict(u=np.ones((1, L, 1)), delta=np.full((1, L, 1), LN2), A=np.array([[-1.0]]),
             Bm=np.ones((1, L, 1)), Cm=np.ones((1, L, 1)), Dskip=None, theta=None,
             lam=None if lam is None else np.full((1, L, 1), lam))
    y, _ = run(p, disc, False)
    return y[0, :, 0]


def test_worked_values_real():
    """N=1, A=-1, delta=ln 2 (alpha = 1/2), B=C=u=1, D=0, derived by hand:
       exp-Euler      y_t = ln2 (2 - 2^-t)
       ZOH            y_t = 1 - 2^-(t+1)        (gamma = expm1(-ln2)/(-1) = 1/2)
       exp-trap 1/2   y_t = ln2 (1.5 - 2^-t)    (b_0 = ln2/2, b_t = 3 ln2/4 after)"""
    t = np.arange(24, dtype=np.float64)
    assert rel_err(_scalar_case("euler"), LN2 * (2 - 2.0 ** -t)) < 1e-15
    assert rel_err(_scalar_case("zoh"), 1 - 2.0 ** -(t + 1)) < 1e-15
    assert rel_err(_scalar_case("trap", 0.5), LN2 * (1.5 - 2.0 ** -t)) < 1e-15


def test_worked_values_rotation():
    """A = 0, theta = pi/2 (alpha = i), exp-Euler, delta = B = u = 1:
       h = 1, 1+i, i, 0, 1, ... (period 4).  C = 1 gives y = 1, 1, 0, 0, ...;
       C = i gives y = 0, -1, -1, 0, ... which fixes e^{+i theta} and no
       conjugate on C (complex state section of the Mamba-3 story page)."""
    L = 16
    p = dict(u=np.ones((1, L, 1)), delta=np.ones((1, L, 1)), A=np.zeros((1, 1)),
             Bm=np.tile([1.0, 0.0], (1, L, 1, 1)), Cm=np.tile([1.0, 0.0], (1, L, 1, 1)), Dskip=None,
             theta=np.full((1, L, 1, 1), math.pi / 2), lam=None)
    y1, h = run(p, "euler", True)
    yi, _ = run(dict(p, Cm=np.tile([0.0, 1.0], (1, L, 1, 1))), "euler", True)
    period = np.array([1, 1, 0, 0] * (L // 4), dtype=np.float64)
    assert np.max(np.abs(y1[0, :, 0] - period)) < 1e-14
    assert np.max(np.abs(yi[0, :, 0] - np.array([0, -1, -1, 0] * (L // 4)))) < 1e-14
    assert np.max(np.abs(h[0, 0, 0] - np.array([0.0, 0.0]))) < 1e-14  # h_15 = h_3 = 0


# ---------------------------------------------------------------- P-h
@pytest.mark.parametrize("disc,cplx", MODES)
def test_continuation_is_bitwise(disc, cplx):
    """Scan [0, L1), then continue from (h, previous q) over [L1, L): identical
    to one scan over [0, L) (the chunk-and-merge view of the chunked scan)."""
    rng = np.random.default_rng(9)
    B, L, D, N, L1 = 2, 45, 3, 4, 17
    p = rand_problem(rng, B, L, D, N, disc, cplx)
    y, h = run(p, disc, cplx)

    def cut(x, a, b, axis=1):
        return None if x is None else np.take(x, range(a, b), axis=axis)

    keys = ["u", "delta", "Bm", "Cm", "theta", "lam"]
    p1 = dict(p, **{k: cut(p[k], 0, L1) for k in keys})
    p2 = dict(p, **{k: cut(p[k], L1, L) for k in keys})
    y1, h1, q1 = run(p1, disc, cplx, return_q=True)
    y2, h2 = run(p2, disc, cplx, h0=h1, q0=q1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, h)


# ---------------------------------------------------------------- P-i
@pytest.mark.parametrize("disc,cplx", MODES)
def test_linearity(disc, cplx):
    """For fixed delta, theta, lambda, A: y is linear in u (skip term included)
    and, with D = 0, linear in B."""
    rng = np.random.default_rng(10)
    p = rand_problem(rng, 1, 30, 2, 3, disc, cplx)
    u2 = rng.normal(size=p["u"].shape)
    ya, _ = run(p, disc, cplx)
    yb, _ = run(dict(p, u=u2), disc, cplx)
    ys, _ = run(dict(p, u=p["u"] + u2), disc, cplx)
    assert rel_err(ys, ya + yb) < 1e-13
    B2 = rng.normal(size=p["Bm"].shape)
    q = dict(p, Dskip=None)
    y1, _ = run(q, disc, cplx)
    y2, _ = run(dict(q, Bm=B2), disc, cplx)
    y12, _ = run(dict(q, Bm=p["Bm"] + B2), disc, cplx)
    assert rel_err(y12, y1 + y2) < 1e-13


# ---------------------------------------------------------------- P-j
def _ode_exact(lmb, nu, T):
    """h(T) for h' = lmb h + sin(nu tau), h(0) = 0 (variation of constants)."""
    e = np.exp(lmb * T)
    return ((np.exp(1j * nu * T) - e) / (1j * nu - lmb) - (np.exp(-1j * nu * T) - e) / (-1j * nu - lmb)) / 2j


@pytest.mark.parametrize("disc,omega,expect", [("euler", 2.0, 2.0), ("zoh", 0.0, 2.0), ("trap", 2.0, 4.0)])
def test_convergence_order(disc, omega, expect):
    """Against the exact ODE solution (independent of the pages' formulas):
    halving delta halves the global error of exp-Euler and ZOH (first order)
    and quarters it for exp-trapezoidal with lambda = 1/2 (second order) --
    the accuracy claims of the discretisation table on the Mamba-3 story page
    and the exponential-integrator view (LTV solution with a transition
    operator) of the metaphor-xennon page, section 3.1.  Step t covers
    [t d, (t+1) d] and takes u_t = f((t+1) d); the forcing vanishes at 0 so the
    h_{-1} = 0, B_{-1}u_{-1} = 0 start is exact."""
    a, nu, T = -0.5, 3.0, 4.0
    cplx = omega != 0.0
    errs = []
    for K in (400, 800, 1600):
        dlt = T / K
        tgrid = (np.arange(K) + 1) * dlt
        p = dict(u=np.sin(nu * tgrid)[None, :, None], delta=np.full((1, K, 1), dlt), A=np.array([[a]]),
                 Bm=np.tile([1.0, 0.0], (1, K, 1, 1)) if cplx else np.ones((1, K, 1)),
                 Cm=np.tile([1.0, 0.0], (1, K, 1, 1)) if cplx else np.ones((1, K, 1)),
                 Dskip=None, theta=np.full((1, K, 1, 1), omega * dlt) if cplx else None,
                 lam=np.full((1, K, 1), 0.5) if disc == "trap" else None)
        _, h = run(p, disc, cplx)
        hT = h[0, 0, 0, 0] + 1j * h[0, 0, 0, 1] if cplx else h[0, 0, 0]
        errs.append(abs(hT - _ode_exact(a + 1j * omega, nu, T)))
    r1, r2 = errs[0] / errs[1], errs[1] / errs[2]
    assert abs(r1 - expect) < 0.1 and abs(r2 - expect) < 0.1, (errs, r1, r2)


# ---------------------------------------------------------------- misc
def test_nan_propagates_and_errors():
    rng = np.random.default_rng(11)
    p = rand_problem(rng, 1, 12, 2, 3, "euler", True)
    p["u"][0, 5, 1] = np.nan
    y, _ = run(p, "euler", True)
    assert np.all(np.isfinite(y[0, :5, 1])) and np.all(np.isnan(y[0, 5:, 1]))
    assert np.all(np.isfinite(y[0, :, 0]))
    with pytest.raises(ValueError):
        run(p, "zoh", True)  # complex ZOH is not defined
    with pytest.raises(ValueError):
        run(dict(p, lam=None), "trap", True)  # trapezoid needs lambda
