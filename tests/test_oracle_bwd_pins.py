"""Pins of the oracle's backward (oracle.scan_bwd) by a route that shares
nothing with it: central finite differences of the fp64 forward oracle.  For
L = sum(dy * y) + sum(dh_last * h_last), every gradient the backward returns
must match (L(x + eps e_i) - L(x - eps e_i)) / (2 eps) for every element i
of every input, for each discretisation, with softplus on and off, and with
one A entry exactly 0 (the ZOH limit branch)."""
import numpy as np
import pytest

import oracle


def _inputs(seed, batch=2, L=9, Dn=3, N=4):
    r = np.random.default_rng(seed)
    x = {
        "u": r.normal(size=(batch, L, Dn)),
        "delta": r.normal(size=(batch, L, Dn)) * 0.5 - 1.0,
        "A": -np.exp(r.uniform(0, 2, size=(Dn, N))),
        "B": r.normal(size=(batch, L, N)),
        "C": r.normal(size=(batch, L, N)),
        "D": r.normal(size=Dn),
        "z": r.normal(size=(batch, L, Dn)),
        "delta_bias": r.normal(size=Dn) * 0.3,
        "h0": r.normal(size=(batch, Dn, N)),
    }
    x["A"][1, 2] = 0.0
    dy = r.normal(size=(batch, L, Dn))
    dh_last = r.normal(size=(batch, Dn, N))
    return x, dy, dh_last


def _loss(x, dy, dh_last, softplus, disc):
    y, hl = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                        delta_bias=x["delta_bias"], h0=x["h0"], softplus=softplus,
                        zoh=disc == "zoh", bilinear=disc == "bilinear")
    return float((dy * y).sum() + (dh_last * hl).sum())


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "z": "dz", "delta_bias": "dbias", "h0": "dh0"}


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "linear"])
@pytest.mark.parametrize("disc", ["euler", "zoh", "bilinear"])
def test_backward_matches_finite_differences(disc, softplus):
    x, dy, dh_last = _inputs(21)
    if not softplus:  # keep dt positive without the softplus
        x["delta"] = np.abs(x["delta"]) * 0.2 + 0.05
        x["delta_bias"] = np.abs(x["delta_bias"]) * 0.1
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                        delta_bias=x["delta_bias"], h0=x["h0"], dh_last=dh_last,
                        softplus=softplus, zoh=disc == "zoh", bilinear=disc == "bilinear")
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        base = x[name]
        num = np.empty_like(base)
        for i in np.ndindex(base.shape):
            keep = base[i]
            base[i] = keep + eps
            lp = _loss(x, dy, dh_last, softplus, disc)
            base[i] = keep - eps
            lm = _loss(x, dy, dh_last, softplus, disc)
            base[i] = keep
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=2e-6, atol=2e-7,
                                   err_msg=f"{gname} ({disc}, softplus={softplus})")


def test_backward_without_optional_terms():
    """No z, D, bias, h0 or dh_last: the gradients of the plain scan still
    match finite differences, and dh0 is the gradient w.r.t. a zero state."""
    x, dy, _ = _inputs(22, L=7)
    for k in ("z", "D", "delta_bias"):
        x[k] = None
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, softplus=True)
    assert g["dz"] is None and g["dD"] is None

    def loss(u):
        y, _ = oracle.scan(u, x["delta"], x["A"], x["B"], x["C"], softplus=True)
        return float((dy * y).sum())

    eps = 1e-6
    u = x["u"].copy()
    num = np.empty_like(u)
    for i in np.ndindex(u.shape):
        keep = u[i]
        u[i] = keep + eps
        lp = loss(u)
        u[i] = keep - eps
        lm = loss(u)
        u[i] = keep
        num[i] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(g["du"], num, rtol=2e-6, atol=2e-7)
