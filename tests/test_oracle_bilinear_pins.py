"""Pins of the oracle's bilinear (Tustin) discretisation against what the
mathematics fixes, none of which retypes the formula:
  * time-invariant inputs give a convolution (numpy.convolve);
  * A = 0 gives the same prefix sum as Euler (numpy.cumsum);
  * the bilinear map keeps the continuous system's DC gain: with u = B = 1 the
    state settles at exactly -1/A (the ODE's equilibrium), which Euler does not;
  * A_bar agrees with exp(dt*A) to third order, with leading error x^3/12
    (x = dt*A), and B_bar with the exact (ZOH) factor to second order, with
    leading error dt*x^2/12 -- a halved or dropped term changes these orders;
  * dt = 0 leaves the state unchanged; split/resume and step == scan hold.
The bilinear transform is the discretisation the intelliparadigm page's
section 3.2 code names (its printed code is garbled)."""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _one_state(dt, a, u=1.0, h0=0.0, bilinear=True, zoh=False, steps=1):
    """Run one channel, one state, C = 1, z/D off: returns h after each step."""
    L = steps
    y, _ = oracle.scan(np.full((1, L, 1), u), np.full((1, L, 1), dt), np.array([[a]]),
                       np.ones((1, L, 1)), np.ones((1, L, 1)), h0=np.array([[[h0]]]),
                       softplus=False, zoh=zoh, bilinear=bilinear)
    return y[0, :, 0]


def test_bilinear_lti_equals_convolution():
    r = _rng(11)
    batch, L, Dn, N = 2, 80, 4, 5
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    dt = np.exp(r.uniform(math.log(1e-3), math.log(3e-1), size=Dn))
    bvec, cvec = r.normal(size=(batch, N)), r.normal(size=(batch, N))
    Dv = r.normal(size=Dn)
    u = r.normal(size=(batch, L, Dn))
    delta = np.broadcast_to(dt, (batch, L, Dn)).copy()
    B = np.broadcast_to(bvec[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(cvec[:, None, :], (batch, L, N)).copy()
    y, _ = oracle.scan(u, delta, A, B, C, D=Dv, softplus=False, bilinear=True)
    # The impulse response of the oracle itself (one unit input at t = 0, no
    # D) gives the kernel; the convolution of u with it must reproduce y.
    for b in range(batch):
        for d in range(Dn):
            imp = np.zeros((1, L, 1))
            imp[0, 0, 0] = 1.0
            K, _ = oracle.scan(imp, delta[b:b + 1, :, d:d + 1], A[d:d + 1], B[b:b + 1],
                               C[b:b + 1], softplus=False, bilinear=True)
            ref = np.convolve(u[b, :, d], K[0, :, 0])[:L] + Dv[d] * u[b, :, d]
            np.testing.assert_allclose(y[b, :, d], ref, rtol=1e-11, atol=1e-12)


def test_bilinear_zero_A_is_prefix_sum():
    r = _rng(12)
    batch, L, Dn, N = 2, 50, 3, 4
    A = np.zeros((Dn, N))
    raw = r.normal(size=(batch, L, Dn))
    u, B, C = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N)])
    y, hl = oracle.scan(u, raw, A, B, C, softplus=True, bilinear=True)
    dt = np.logaddexp(0.0, raw)
    h = np.cumsum(dt[:, :, :, None] * B[:, :, None, :] * u[:, :, :, None], axis=1)
    np.testing.assert_allclose(y, (h * C[:, :, None, :]).sum(-1), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hl, h[:, -1], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("a", [-0.5, -3.0, -20.0])
@pytest.mark.parametrize("dt", [0.01, 0.3, 2.0])
def test_bilinear_keeps_the_dc_gain(a, dt):
    """u = B = 1: the ODE h' = a h + 1 settles at -1/a.  The bilinear state
    settles there too, to rounding (Euler does not unless dt -> 0)."""
    # Long enough for the transient to die out below 1e-16: a stiff step
    # (abs(dt*a) >> 2) gives an A_bar near -1, which decays slowly.
    x = dt * a
    rate = abs((1 + x / 2) / (1 - x / 2))
    steps = int(math.ceil(37.0 / -math.log(rate))) + 10
    h = _one_state(dt, a, steps=steps)
    assert abs(h[-1] - (-1.0 / a)) <= 1e-12 * (1.0 / abs(a))
    h_euler = _one_state(dt, a, steps=steps, bilinear=False)
    if dt * abs(a) > 0.05:
        assert abs(h_euler[-1] - (-1.0 / a)) > 1e-4 * (1.0 / abs(a))


@pytest.mark.parametrize("x", [-1e-2, -3e-3, -1e-3])
def test_bilinear_abar_is_third_order_accurate(x):
    """One step from h0 = 1 with u = 0 returns A_bar; (A_bar - e^x)/x^3 -> 1/12."""
    a = -2.0
    dt = x / a
    abar = _one_state(dt, a, u=0.0, h0=1.0)[0]
    ratio = (abar - math.exp(x)) / x ** 3
    assert abs(ratio - 1.0 / 12.0) < 0.02 * (1.0 / 12.0) + abs(x)


@pytest.mark.parametrize("x", [-1e-2, -3e-3])
def test_bilinear_bbar_is_second_order_accurate(x):
    """One step from h0 = 0 with u = B = 1 returns B_bar; against the exact
    (ZOH) factor, (B_bar - B_zoh)/(dt x^2) -> 1/12."""
    a = -4.0
    dt = x / a
    bb = _one_state(dt, a)[0]
    bz = _one_state(dt, a, bilinear=False, zoh=True)[0]
    ratio = (bb - bz) / (dt * x * x)
    assert abs(ratio - 1.0 / 12.0) < 0.02 * (1.0 / 12.0) + abs(x)


def test_bilinear_zero_step_split_and_decode():
    r = _rng(13)
    batch, L, Dn, N = 2, 30, 3, 4
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    u, B, C, z = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N),
                                             (batch, L, Dn)])
    h0 = r.normal(size=(batch, Dn, N))
    # dt = 0: identity
    _, hl = oracle.scan(u, np.zeros((batch, L, Dn)), A, B, C, h0=h0, softplus=False,
                        bilinear=True)
    np.testing.assert_array_equal(hl, h0)
    raw = r.normal(size=(batch, L, Dn))
    y, hl = oracle.scan(u, raw, A, B, C, z=z, h0=h0, softplus=True, bilinear=True)
    # split / resume
    L1 = 13
    y1, h1 = oracle.scan(u[:, :L1], raw[:, :L1], A, B[:, :L1], C[:, :L1], z=z[:, :L1], h0=h0,
                         softplus=True, bilinear=True)
    y2, h2 = oracle.scan(u[:, L1:], raw[:, L1:], A, B[:, L1:], C[:, L1:], z=z[:, L1:], h0=h1,
                         softplus=True, bilinear=True)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h2, hl, rtol=1e-13, atol=1e-13)
    # decode steps == scan
    h = h0
    for t in range(L):
        yt, h = oracle.step(h, u[:, t], raw[:, t], A, B[:, t], C[:, t], z=z[:, t],
                            softplus=True, bilinear=True)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h, hl, rtol=1e-13, atol=1e-13)
