"""Accuracy and bias of the scan kernel's transcendental policies on the GPU.

The library applies the chunked kernel's own inline exp and sin/cos
functions (csrc/device_math.h) element-wise through
ssm_calibrate_device_math, over the argument ranges of the workloads' input
recipe:
  * exp(delta A): delta = softplus(N(mu, 0.5)) for mu in {-4, -3, -2},
    A = -exp(U(-3, 0)) (complex workloads) or -(n + 1), n < 16 (real ZOH);
  * the rotation angle theta = s * U(-pi, pi), s = 0.1 (the workloads) and
    s = 1, 30 and 10^4 (the wide-angle parity cases);
  * the ZOH weight's e^z - 1 and e^z at z = delta A.
The reference is fp64 (numpy) on the same fp32 arguments.  Errors are in
units of the fp32 spacing at the reference value (ulp) for exp, e^z - 1 and
the fp32 path's sin/cos, and in units of 2^-24 (half an ulp at 1) absolute
for the hardware sin/cos, whose error is absolute: they rotate a state of
modulus |alpha|, so an absolute error is what enters the recurrence.  The
mean signed error is the bias that compounds over a slowly decaying state;
the bounds below are the measured figures with margin.
"""
import math

import numpy as np
import pytest
import torch

from selective_state_space_42_amd import scan

pytestmark = pytest.mark.gpu

N = 1 << 20


def _softplus(v):
    return np.log1p(np.exp(v))


def _ulp_err(got, ref):
    """Signed error of fp32 results in ulps of the fp32 reference value."""
    ref32 = ref.astype(np.float32)
    spacing = np.spacing(np.abs(ref32)).astype(np.float64)
    return (got.astype(np.float64) - ref) / spacing


def _run(fn, x, y=None):
    xt = torch.from_numpy(x.astype(np.float32)).cuda()
    yt = torch.from_numpy(y.astype(np.float32)).cuda() if y is not None else None
    out = scan.ssm_calibrate_device_math(fn, xt, yt)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _delta_A(rng, mu, a_kind):
    delta = _softplus(rng.normal(mu, 0.5, N)).astype(np.float32)
    if a_kind == "neg_exp_uniform":
        A = (-np.exp(rng.uniform(-3.0, 0.0, N))).astype(np.float32)
    else:
        A = (-(rng.integers(0, 16, N) + 1)).astype(np.float32)
    return delta, A


@pytest.mark.parametrize("mu,a_kind", [(-4.0, "neg_exp_uniform"), (-3.0, "neg_exp_uniform"),
                                       (-3.0, "neg_index"), (-2.0, "neg_exp_uniform")])
def test_exp_delta_A(mu, a_kind):
    rng = np.random.default_rng(11)
    delta, A = _delta_A(rng, mu, a_kind)
    got = _run("exp_dA", delta, A)
    z = delta.astype(np.float64) * A.astype(np.float64)
    e = _ulp_err(got, np.exp(z))
    # the argument delta * (A log2 e) is rounded twice in fp32, a relative
    # error of up to 2^-23 in the exponent, i.e. |z| 2^-23 in the result:
    # up to 2 |z| ulp on top of the hardware 2^x's own error
    excess = np.abs(e) - 2.0 * np.abs(z)
    print(f"exp(delta A) mu={mu} {a_kind}: mean {e.mean():+.4f} ulp, max |err| {np.abs(e).max():.2f} ulp, "
          f"max |err| - 2|z| {excess.max():.2f} ulp, max |z| {np.abs(z).max():.2f}")
    assert abs(e.mean()) < 0.1
    assert excess.max() < 1.5


@pytest.mark.parametrize("scale", [0.1, 1.0, 30.0])
def test_hardware_sin_cos(scale):
    rng = np.random.default_rng(12)
    th = (scale * rng.uniform(-math.pi, math.pi, N)).astype(np.float32)
    t64 = th.astype(np.float64)
    unit = 2.0 ** -24
    es = (_run("sin_hw", th).astype(np.float64) - np.sin(t64)) / unit
    ec = (_run("cos_hw", th).astype(np.float64) - np.cos(t64)) / unit
    print(f"hardware sin/cos, theta = {scale} U(-pi, pi): sin mean {es.mean():+.3f} max {np.abs(es).max():.2f}, "
          f"cos mean {ec.mean():+.3f} max {np.abs(ec).max():.2f} (units of 2^-24)")
    # the fract(theta / 2 pi) in fp32 adds |theta| * 2^-24-sized argument error at wide angles
    lim = 8.0 + 4.0 * scale * math.pi
    assert np.abs(es).max() < lim and np.abs(ec).max() < lim
    assert abs(es.mean()) < 0.5 and abs(ec.mean()) < 1.5


def test_polynomial_sin_cos_quarter_turn():
    rng = np.random.default_rng(13)
    th = rng.uniform(-math.pi / 4, math.pi / 4, N).astype(np.float32)
    t64 = th.astype(np.float64)
    keep = np.abs(t64) > 1e-3  # sin's ulp shrinks with the value; near 0 it is x itself
    es = _ulp_err(_run("sin_poly", th), np.sin(t64))[keep]
    ec = _ulp_err(_run("cos_poly", th), np.cos(t64))
    print(f"polynomial sin/cos on |theta| <= pi/4: sin mean {es.mean():+.4f} max {np.abs(es).max():.2f}, "
          f"cos mean {ec.mean():+.4f} max {np.abs(ec).max():.2f} ulp")
    assert np.abs(es).max() < 1.5 and np.abs(ec).max() < 1.5
    assert abs(es.mean()) < 0.1 and abs(ec.mean()) < 0.1


@pytest.mark.parametrize("scale", [1.0, 30.0, 1e4])
def test_wide_sin_cos(scale):
    rng = np.random.default_rng(14)
    th = (scale * rng.uniform(-math.pi, math.pi, N)).astype(np.float32)
    t64 = th.astype(np.float64)
    s, c = np.sin(t64), np.cos(t64)
    ks, kc = np.abs(s) > 1e-3, np.abs(c) > 1e-3
    es = _ulp_err(_run("sin_wide", th), s)[ks]
    ec = _ulp_err(_run("cos_wide", th), c)[kc]
    print(f"reduced sin/cos, theta = {scale} U(-pi, pi): sin mean {es.mean():+.4f} max {np.abs(es).max():.2f}, "
          f"cos mean {ec.mean():+.4f} max {np.abs(ec).max():.2f} ulp")
    assert np.abs(es).max() < 2.0 and np.abs(ec).max() < 2.0
    assert abs(es.mean()) < 0.1 and abs(ec.mean()) < 0.1


@pytest.mark.parametrize("mu", [-3.0, -2.0])
def test_zoh_weight_terms(mu):
    rng = np.random.default_rng(15)
    delta, A = _delta_A(rng, mu, "neg_index")
    z = delta.astype(np.float64) * A.astype(np.float64)
    em1 = _ulp_err(_run("expm1_zoh", delta, A), np.expm1(z))
    ez = _ulp_err(_run("exp_zoh", delta, A), np.exp(z))
    small = np.abs(z) <= math.log(2) / 2  # the polynomial's range
    # outside it both come from the hardware 2^x of a twice-rounded exponent
    # (see test_exp_delta_A); e^z - 1 = e^z - 1 adds at most e^z / |e^z - 1| < 2.5 times that
    print(f"ZOH mu={mu}: polynomial range {small.mean():.1%} of the arguments; e^z - 1 there mean "
          f"{em1[small].mean():+.4f} max {np.abs(em1[small]).max():.2f} ulp; elsewhere max |err| - 5|z| "
          f"{(np.abs(em1[~small]) - 5 * np.abs(z[~small])).max():.2f}; e^z max |err| - 2|z| "
          f"{(np.abs(ez) - 2 * np.abs(z)).max():.2f} ulp")
    assert np.abs(em1[small]).max() < 2.5 and abs(em1[small].mean()) < 0.2
    assert (np.abs(em1[~small]) - 5 * np.abs(z[~small])).max() < 4.0
    assert (np.abs(ez) - 2 * np.abs(z)).max() < 1.5
