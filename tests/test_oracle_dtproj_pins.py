"""Pins of the oracle's fused-projection scan (oracle.scan_dtproj) against
routes that share nothing with its matrix product:
  * a 0/1 selection weight W[d, r] = [r == (d + s) mod rank] makes the raw
    step of channel d the column (d + s) mod rank of dt_low, picked by numpy
    indexing, so the result must equal the pinned plain scan on that delta.
    A square case (rank = d_inner, shift s = 1) tells W from its transpose;
  * a rank-1 weight gives the outer product dt_low[..., 0] * w[d]
    (numpy broadcasting);
  * permuting the rank columns of dt_low and W together changes nothing, and
    a zero weight gives the scan with delta = bias only.
The plain scan these reduce to is pinned on its own (closed forms, brute
force, the worked example)."""
import numpy as np
import pytest

import oracle


def _inputs(seed, batch=2, L=40, Dn=6, N=4, rank=3):
    r = np.random.default_rng(seed)
    return {
        "u": r.normal(size=(batch, L, Dn)),
        "dt_low": r.normal(size=(batch, L, rank)) * 0.7,
        "A": -np.exp(r.uniform(0, 2, size=(Dn, N))),
        "B": r.normal(size=(batch, L, N)),
        "C": r.normal(size=(batch, L, N)),
        "D": r.normal(size=Dn),
        "z": r.normal(size=(batch, L, Dn)),
        "delta_bias": r.normal(size=Dn) * 0.3,
        "h0": r.normal(size=(batch, Dn, N)),
    }


def _both(x, W, delta, disc):
    kw = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"], softplus=True,
              zoh=disc == "zoh", bilinear=disc == "bilinear")
    got = oracle.scan_dtproj(x["u"], x["dt_low"], W, x["A"], x["B"], x["C"], **kw)
    ref = oracle.scan(x["u"], delta, x["A"], x["B"], x["C"], **kw)
    return got, ref


@pytest.mark.parametrize("disc", ["euler", "zoh", "bilinear"])
@pytest.mark.parametrize("Dn,rank,shift", [(6, 3, 0), (6, 3, 2), (5, 5, 1), (4, 7, 3)])
def test_selection_weight_picks_columns(disc, Dn, rank, shift):
    x = _inputs(41 + Dn + rank, Dn=Dn, rank=rank)
    W = np.zeros((Dn, rank))
    cols = (np.arange(Dn) + shift) % rank
    W[np.arange(Dn), cols] = 1.0
    delta = x["dt_low"][:, :, cols]
    (y, hl), (yr, hr) = _both(x, W, delta, disc)
    np.testing.assert_allclose(y, yr, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hl, hr, rtol=1e-13, atol=1e-13)


def test_selection_tells_w_from_its_transpose():
    """rank == d_inner with a shift: using W^T would pick column d - 1."""
    x = _inputs(50, Dn=5, rank=5)
    W = np.zeros((5, 5))
    W[np.arange(5), (np.arange(5) + 1) % 5] = 1.0
    y, _ = oracle.scan_dtproj(x["u"], x["dt_low"], W, x["A"], x["B"], x["C"], softplus=True)
    y_t, _ = oracle.scan_dtproj(x["u"], x["dt_low"], W.T, x["A"], x["B"], x["C"], softplus=True)
    yr, _ = oracle.scan(x["u"], x["dt_low"][:, :, (np.arange(5) + 1) % 5], x["A"], x["B"],
                        x["C"], softplus=True)
    np.testing.assert_allclose(y, yr, rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(y_t - yr)) > 1e-3


@pytest.mark.parametrize("disc", ["euler", "zoh"])
def test_rank_one_is_an_outer_product(disc):
    x = _inputs(51, rank=1)
    w = np.random.default_rng(52).normal(size=6)
    delta = x["dt_low"][:, :, :1] * w[None, None, :]
    (y, hl), (yr, hr) = _both(x, w[:, None], delta, disc)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hl, hr, rtol=1e-12, atol=1e-12)


def test_column_permutation_and_zero_weight():
    x = _inputs(53, rank=4)
    W = np.random.default_rng(54).normal(size=(6, 4)) * 0.5
    perm = np.array([2, 0, 3, 1])
    y, _ = oracle.scan_dtproj(x["u"], x["dt_low"], W, x["A"], x["B"], x["C"],
                              delta_bias=x["delta_bias"], softplus=True)
    yp, _ = oracle.scan_dtproj(x["u"], x["dt_low"][:, :, perm], W[:, perm], x["A"], x["B"],
                               x["C"], delta_bias=x["delta_bias"], softplus=True)
    np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-12)
    y0, _ = oracle.scan_dtproj(x["u"], x["dt_low"], np.zeros((6, 4)), x["A"], x["B"], x["C"],
                               delta_bias=x["delta_bias"], softplus=True)
    yb, _ = oracle.scan(x["u"], np.zeros(x["u"].shape), x["A"], x["B"], x["C"],
                        delta_bias=x["delta_bias"], softplus=True)
    np.testing.assert_allclose(y0, yb, rtol=1e-13, atol=1e-13)
