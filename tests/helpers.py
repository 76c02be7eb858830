"""Shared pieces of the GPU parity tests: tolerances and sampled comparisons.

Tolerances (stated for this path):
  fp32 io : |err| <= 1e-4 * (1 + |ref|)
  bf16 io : |err| <= 2 ulp_bf16(ref) + 1e-3, ulp_bf16(v) = 2^(floor(log2|v|) - 7),
            against the fp64 oracle run on the same bf16-rounded inputs.
  fp32 state (h_last, decode h): |err| <= 1e-4 * (1 + |ref|).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def bound(ref: np.ndarray, io: str) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    if io == "f32":
        return 1e-4 * (1.0 + np.abs(ref))
    a = np.abs(ref)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a > 0, np.exp2(e - 7.0), 0.0)
    return 2.0 * ulp + 1e-3


def assert_within(got, ref, io: str, what: str = "y"):
    got = got.detach().to("cpu").double().numpy() if hasattr(got, "detach") else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = bound(ref, io)
    bad = ~(err <= lim)           # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        worst = float(np.nanmax(np.where(np.isfinite(err), err / lim, np.inf)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the bound "
                             f"(worst err/bound {worst:.3g}); first at {idx.tolist()}: "
                             f"got {[float(got[tuple(i)]) for i in idx]} "
                             f"ref {[float(ref[tuple(i)]) for i in idx]}")
    return float(np.max(err / lim)) if err.size else 0.0


def sample_channels(Dn: int, k: int, seed: int = 0) -> np.ndarray:
    """k channel indices covering both ends, tile edges and random picks."""
    must = sorted({0, Dn - 1, min(63, Dn - 1), min(64, Dn - 1)})
    rng = np.random.default_rng(seed)
    rest = [int(i) for i in rng.permutation(Dn) if int(i) not in must]
    idx = must + rest[:max(0, k - len(must))]
    return np.array(sorted(idx), dtype=np.int64)


def disc_kw(disc: str) -> dict:
    """Keyword arguments of scan_fwd / oracle.scan for a discretisation name."""
    assert disc in ("euler", "zoh", "bilinear"), disc
    return {"zoh": disc == "zoh", "bilinear": disc == "bilinear"}


DISCS = ["euler", "zoh", "bilinear"]


def oracle_on_channels(x: dict, idx: np.ndarray, softplus: bool, zoh: bool,
                       h0: torch.Tensor | None = None, bilinear: bool = False):
    """Run the oracle on a subset of channels (all batches, full L).  Channels
    are independent, so this is exactly the full oracle restricted to them."""
    ii = torch.as_tensor(idx, device=x["u"].device)
    sub = {
        "u": x["u"].index_select(2, ii), "delta": x["delta"].index_select(2, ii),
        "z": x["z"].index_select(2, ii) if "z" in x and x["z"] is not None else None,
        "B": x["B"], "C": x["C"],
        "A": x["A"].index_select(0, ii),
        "D": x["D"].index_select(0, ii) if x.get("D") is not None else None,
        "delta_bias": x["delta_bias"].index_select(0, ii) if x.get("delta_bias") is not None
        else None,
    }
    h0s = h0.index_select(1, ii) if h0 is not None else None
    return oracle.scan(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], D=sub["D"],
                       z=sub["z"], delta_bias=sub["delta_bias"], h0=h0s, softplus=softplus,
                       zoh=zoh, bilinear=bilinear)
