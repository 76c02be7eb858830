"""Pins of the fp64 oracle against what the pages and mathematics fix.

None of these re-types the oracle's loop: each compares it with a different
route to the same number -- a convolution (the linear time-invariant case),
a prefix sum (A = 0), explicit products of decays, a closed-form ODE step
response (zero-order hold), a geometric series (Euler), a hand-worked example,
or structural identities (split/resume, step == scan, linearity).  Library
routines used as independent references: numpy.convolve, numpy.cumsum,
numpy.logaddexp, scipy.special.expit.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

RTOL = 1e-12


def _close(a, b, rtol=RTOL, atol=1e-13):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def _rng(seed):
    return np.random.default_rng(seed)


def _silu(z):
    return z * expit(z)


# ---------------------------------------------------------------- P-1: LTI ---
# With dt, B, C fixed over time the system is time invariant, so the output is
# a causal convolution of u with K_j = sum_n c_n abar_n^j bbar_n (lmnt page
# section 2.1: fixed A, B, C give an LTI system computable by convolution).
@pytest.mark.parametrize("zoh", [False, True])
def test_lti_equals_convolution(zoh):
    r = _rng(1)
    batch, L, Dn, N = 2, 97, 5, 6
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    dt = np.exp(r.uniform(math.log(1e-3), math.log(3e-1), size=Dn))  # per channel
    bvec = r.normal(size=(batch, N))
    cvec = r.normal(size=(batch, N))
    Dv = r.normal(size=Dn)
    u = r.normal(size=(batch, L, Dn))
    delta = np.broadcast_to(dt, (batch, L, Dn)).copy()
    B = np.broadcast_to(bvec[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(cvec[:, None, :], (batch, L, N)).copy()
    y, _ = oracle.scan(u, delta, A, B, C, D=Dv, softplus=False, zoh=zoh)
    for b in range(batch):
        for d in range(Dn):
            abar = np.exp(dt[d] * A[d])
            if zoh:
                bfac = np.expm1(dt[d] * A[d]) / A[d]
            else:
                bfac = np.full(N, dt[d])
            j = np.arange(L)[:, None]
            K = (cvec[b] * bvec[b] * bfac * abar ** j).sum(axis=1)
            ref = np.convolve(u[b, :, d], K)[:L] + Dv[d] * u[b, :, d]
            _close(y[b, :, d], ref, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------- P-2: prefix sum ---
# A = 0 makes every decay 1, so the state is a running sum of dt_k B_k u_k.
# The ZOH factor takes its limit dt at A = 0 (reading R3), so both agree.
@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("softplus", [False, True])
def test_zero_A_is_prefix_sum(zoh, softplus):
    r = _rng(2)
    batch, L, Dn, N = 3, 64, 4, 5
    A = np.zeros((Dn, N))
    raw = r.normal(size=(batch, L, Dn)) * (1.0 if softplus else 0.05) + (0 if softplus else 0.1)
    bias = r.normal(size=Dn) * 0.5
    u, B, C, z = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N),
                                             (batch, L, Dn)])
    Dv = r.normal(size=Dn)
    y, hl = oracle.scan(u, raw, A, B, C, D=Dv, z=z, delta_bias=bias,
                        softplus=softplus, zoh=zoh)
    dt = raw + bias
    if softplus:
        dt = np.logaddexp(0.0, dt)          # log(1 + e^x), library routine
    incr = dt[:, :, :, None] * B[:, :, None, :] * u[:, :, :, None]   # [b,t,d,n]
    h = np.cumsum(incr, axis=1)
    yref = (h * C[:, :, None, :]).sum(-1) + Dv * u
    yref = yref * _silu(z)
    _close(y, yref, rtol=1e-11, atol=1e-12)
    _close(hl, h[:, -1], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------ P-3: brute force ---
# h_t = sum_k (prod_{j=k+1..t} abar_j) bbar_k u_k, by explicit products and
# again with the products folded into one exponential exp(A * sum dt_j)
# (jsqmd page section 3.4: composing the per-step affine maps).
@pytest.mark.parametrize("zoh", [False, True])
def test_brute_force_unrolling(zoh):
    r = _rng(3)
    batch, L, Dn, N = 1, 11, 2, 3
    A = -np.exp(r.uniform(0, 2, size=(Dn, N)))
    raw = r.normal(size=(batch, L, Dn))
    u, B, C = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N)])
    y, hl = oracle.scan(u, raw, A, B, C, softplus=True, zoh=zoh)
    dt = np.logaddexp(0.0, raw)
    for d in range(Dn):
        for t in range(L):
            yt = 0.0
            for n in range(N):
                a = A[d, n]
                h_prod = 0.0
                h_exp = 0.0
                for k in range(t + 1):
                    p = 1.0
                    for j in range(k + 1, t + 1):
                        p *= math.exp(dt[0, j, d] * a)
                    bf = (math.expm1(dt[0, k, d] * a) / a) if zoh else dt[0, k, d]
                    term = bf * B[0, k, n] * u[0, k, d]
                    h_prod += p * term
                    h_exp += math.exp(a * dt[0, k + 1:t + 1, d].sum()) * term
                assert abs(h_prod - h_exp) <= 1e-12 * (1 + abs(h_prod))
                yt += C[0, t, n] * h_prod
                if t == L - 1:
                    assert abs(hl[0, d, n] - h_prod) <= 1e-12 * (1 + abs(h_prod))
            assert abs(y[0, t, d] - yt) <= 1e-12 * (1 + abs(yt))


# ------------------------------------------------------------ P-4: dt -> 0 ---
# dt = 0 gives abar = 1 and bbar = 0: the state never moves, and
# y_t = (C_t . h0 + D u_t) * silu(z_t).
@pytest.mark.parametrize("zoh", [False, True])
def test_zero_step_keeps_state(zoh):
    r = _rng(4)
    batch, L, Dn, N = 2, 20, 3, 4
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    raw = np.zeros((batch, L, Dn))
    u, B, C, z = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N),
                                             (batch, L, Dn)])
    Dv = r.normal(size=Dn)
    h0 = r.normal(size=(batch, Dn, N))
    y, hl = oracle.scan(u, raw, A, B, C, D=Dv, z=z, h0=h0, softplus=False, zoh=zoh)
    _close(hl, h0, rtol=0, atol=0)
    ref = (np.einsum("btn,bdn->btd", C, h0) + Dv * u) * _silu(z)
    _close(y, ref, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- P-5: split/resume ---
@pytest.mark.parametrize("zoh", [False, True])
def test_split_resume_equals_one_scan(zoh):
    r = _rng(5)
    batch, L, Dn, N = 2, 50, 3, 5
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    raw = r.normal(size=(batch, L, Dn)) - 2
    u, B, C, z = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N),
                                             (batch, L, Dn)])
    Dv, bias = r.normal(size=Dn), r.normal(size=Dn) * 0.1
    kw = dict(D=Dv, delta_bias=bias, softplus=True, zoh=zoh)
    y, hl = oracle.scan(u, raw, A, B, C, z=z, **kw)
    for L1 in (1, 17, 49):
        y1, h1 = oracle.scan(u[:, :L1], raw[:, :L1], A, B[:, :L1], C[:, :L1], z=z[:, :L1], **kw)
        y2, h2 = oracle.scan(u[:, L1:], raw[:, L1:], A, B[:, L1:], C[:, L1:], z=z[:, L1:],
                             h0=h1, **kw)
        _close(np.concatenate([y1, y2], axis=1), y, rtol=1e-13, atol=1e-14)
        _close(h2, hl, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------- P-6: step == scan ---
@pytest.mark.parametrize("zoh", [False, True])
def test_decode_steps_equal_scan(zoh):
    r = _rng(6)
    batch, L, Dn, N = 2, 9, 4, 3
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    raw = r.normal(size=(batch, L, Dn)) - 2
    u, B, C, z = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N),
                                             (batch, L, Dn)])
    Dv = r.normal(size=Dn)
    h0 = r.normal(size=(batch, Dn, N))
    y, hl = oracle.scan(u, raw, A, B, C, D=Dv, z=z, h0=h0, softplus=True, zoh=zoh)
    h = h0
    for t in range(L):
        yt, h = oracle.step(h, u[:, t], raw[:, t], A, B[:, t], C[:, t], D=Dv, z=z[:, t],
                            softplus=True, zoh=zoh)
        _close(yt, y[:, t], rtol=0, atol=0)
    _close(h, hl, rtol=0, atol=0)


# -------------------------------------------------------- P-7: linearity ---
@pytest.mark.parametrize("zoh", [False, True])
def test_linear_in_u_and_affine_in_h0(zoh):
    r = _rng(7)
    batch, L, Dn, N = 2, 40, 3, 4
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    raw = r.normal(size=(batch, L, Dn)) - 2
    B, C, z = (r.normal(size=s) for s in [(batch, L, N), (batch, L, N), (batch, L, Dn)])
    Dv = r.normal(size=Dn)
    u1, u2 = r.normal(size=(batch, L, Dn)), r.normal(size=(batch, L, Dn))
    kw = dict(D=Dv, z=z, softplus=True, zoh=zoh)
    a, b = 0.75, -1.5
    y12, _ = oracle.scan(a * u1 + b * u2, raw, A, B, C, **kw)
    y1, _ = oracle.scan(u1, raw, A, B, C, **kw)
    y2, _ = oracle.scan(u2, raw, A, B, C, **kw)
    _close(y12, a * y1 + b * y2, rtol=1e-11, atol=1e-12)
    h1, h2 = r.normal(size=(batch, Dn, N)), r.normal(size=(batch, Dn, N))
    y0, _ = oracle.scan(u1, raw, A, B, C, **kw)
    ya, _ = oracle.scan(u1, raw, A, B, C, h0=h1, **kw)
    yb, _ = oracle.scan(u1, raw, A, B, C, h0=h2, **kw)
    yab, _ = oracle.scan(u1, raw, A, B, C, h0=h1 + h2, **kw)
    _close(yab - y0, (ya - y0) + (yb - y0), rtol=1e-10, atol=1e-12)


# ----------------------------------------- P-9: ZOH is the exact ODE step ---
# With u = B = 1 the continuous state obeys h' = A h + 1, whose exact value
# after total time T from h = 0 is expm1(A T)/A.  The zero-order-hold form
# reproduces it for any step sizes; the Euler form dt*B does not.
def test_zoh_reproduces_exact_step_response():
    r = _rng(9)
    batch, L, Dn, N = 1, 300, 3, 8
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    dt = np.exp(r.uniform(math.log(1e-3), math.log(2e-1), size=(batch, L, Dn)))
    u = np.ones((batch, L, Dn))
    B = np.ones((batch, L, N))
    C = np.zeros((batch, L, N))
    for Lc in (1, 7, 300):
        _, hz = oracle.scan(u[:, :Lc], dt[:, :Lc], A, B[:, :Lc], C[:, :Lc], softplus=False,
                            zoh=True)
        _, he = oracle.scan(u[:, :Lc], dt[:, :Lc], A, B[:, :Lc], C[:, :Lc], softplus=False,
                            zoh=False)
        T = dt[0, :Lc].sum(axis=0)                     # [Dn]
        exact = np.expm1(A * T[:, None]) / A
        _close(hz[0], exact, rtol=1e-12, atol=1e-15)
        # Euler's bbar = dt differs from the exact response by O(dt).
        assert np.max(np.abs(he[0] - exact)) > 1e-6


# -------------------------------- Euler with fixed dt: geometric series ---
def test_euler_fixed_step_geometric_series():
    batch, L, Dn, N = 1, 33, 2, 3
    A = -np.array([[0.5, 1.0, 7.0], [2.0, 3.0, 11.0]])
    dt = np.array([0.05, 0.2])
    u = np.ones((batch, L, Dn))
    B = np.ones((batch, L, N))
    C = np.zeros((batch, L, N))
    delta = np.broadcast_to(dt, (batch, L, Dn)).copy()
    _, h = oracle.scan(u, delta, A, B, C, softplus=False, zoh=False)
    a = np.exp(dt[:, None] * A)
    ref = dt[:, None] * (1 - a ** L) / (1 - a)
    _close(h[0], ref, rtol=1e-12)


# ----------------------------------------- bias placement and softplus form ---
def test_bias_inside_softplus_and_zero_bias_equals_none():
    r = _rng(10)
    batch, L, Dn, N = 1, 30, 4, 2
    A = -np.exp(r.uniform(0, 3, size=(Dn, N)))
    raw = r.normal(size=(batch, L, Dn))
    u, B, C = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N)])
    bias = r.normal(size=Dn)
    y_b, _ = oracle.scan(u, raw, A, B, C, delta_bias=bias, softplus=True)
    y_shift, _ = oracle.scan(u, raw + bias, A, B, C, softplus=True)
    _close(y_b, y_shift, rtol=1e-13, atol=1e-14)
    y0, _ = oracle.scan(u, raw, A, B, C, delta_bias=np.zeros(Dn), softplus=True)
    yn, _ = oracle.scan(u, raw, A, B, C, softplus=True)
    _close(y0, yn, rtol=0, atol=0)
    # Extreme raw values: softplus must neither overflow nor lose small steps.
    for v in (-40.0, -12.0, 0.0, 30.0, 700.0):
        rawc = np.full((1, 1, 1), v)
        yv, hv = oracle.scan(np.ones((1, 1, 1)), rawc, np.zeros((1, 1)), np.ones((1, 1, 1)),
                             np.ones((1, 1, 1)), softplus=True)
        want = np.logaddexp(0.0, v)
        assert abs(hv[0, 0, 0] - want) <= 1e-15 * max(1.0, abs(want)) + 1e-300


# --------------------------------------- hand-worked golden example ---
def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = [float(x) for x in v.split()]
    return vals


@pytest.mark.parametrize("zoh", [False, True])
def test_hand_worked_example(zoh):
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "halving_example.txt"))
    L = len(g["u"])
    u = np.array(g["u"]).reshape(1, L, 1)
    B = np.array(g["B"]).reshape(1, L, 1)
    C = np.array(g["C"]).reshape(1, L, 1)
    delta = np.array(g["delta"]).reshape(1, L, 1)
    A = np.array([[-math.log(2.0)]])
    Dv = np.array(g["D"])
    y, h = oracle.scan(u, delta, A, B, C, D=Dv, softplus=False, zoh=zoh)
    key = "zoh" if zoh else "euler"
    _close(y[0, :, 0], np.array(g[f"y_{key}"]), rtol=1e-15, atol=1e-15)
    _close(h[0, 0, 0], g[f"h_last_{key}"][0], rtol=1e-15, atol=1e-15)


# --------------------------- mutation check: the pins catch planted errors ---
def test_pins_would_catch_a_dropped_skip_term():
    """A planted mistake on the CPU side: dropping D from the oracle's output
    must break the prefix-sum pin.  (Done by comparing against a reference
    with D present; the oracle run omits D.)"""
    r = _rng(11)
    batch, L, Dn, N = 1, 8, 2, 2
    u, B, C = (r.normal(size=s) for s in [(batch, L, Dn), (batch, L, N), (batch, L, N)])
    raw = np.full((batch, L, Dn), 0.1)
    Dv = np.array([1.5, -2.0])
    y_noD, _ = oracle.scan(u, raw, np.zeros((Dn, N)), B, C, softplus=False)
    h = np.cumsum(0.1 * B[:, :, None, :] * u[:, :, :, None], axis=1)
    ref = (h * C[:, :, None, :]).sum(-1) + Dv * u
    assert np.max(np.abs(y_noD - ref)) > 1e-3
