"""The seeded input generator: determinism, ranges, and P-8 (softplus of the
inverse softplus returns the drawn step size)."""
import math

import numpy as np
import torch

import synth


def test_same_seed_same_bytes_and_streams_independent():
    w = synth.workload("tiny", L=64)
    a = synth.scan_inputs(w, seed=0)
    b = synth.scan_inputs(w, seed=0)
    c = synth.scan_inputs(w, seed=1)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["u"], c["u"])
    # Per-tensor streams: u and z differ although drawn alike.
    assert not torch.equal(a["u"], a["z"])


def test_step_size_range_roundtrip():
    # softplus(softplus^-1(x)) == x on the log-uniform range [1e-3, 1e-1].
    w = synth.workload("tiny", L=512)
    x = synth.scan_inputs(w, seed=3)["delta"].double().numpy()
    dt = np.logaddexp(0.0, x)
    assert dt.min() >= 1e-3 * (1 - 1e-6) and dt.max() <= 1e-1 * (1 + 1e-6)
    # log-uniform: about half the mass below the geometric mean 1e-2
    frac = float((dt < 1e-2).mean())
    assert 0.45 < frac < 0.55
    v = torch.tensor([1e-3, 3e-3, 1e-2, 5e-2, 1e-1], dtype=torch.float64)
    back = torch.nn.functional.softplus(synth.softplus_inverse(v))
    assert torch.allclose(back, v, rtol=1e-12, atol=0)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1).
    t = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    r = t.to(torch.bfloat16).float().tolist()
    assert r == [1.0, 1.0 + 2 ** -6, -1.0]


def test_workload_shapes_and_a_init():
    w = synth.workload("m130m", batch=1, L=8, Dn=64)
    x = synth.scan_inputs(w)
    assert x["u"].dtype == torch.bfloat16 and x["u"].shape == (1, 8, 64)
    assert x["B"].shape == (1, 8, 16) and x["A"].shape == (64, 16)
    a = x["A"][0].double()
    assert math.isclose(float(a[0]), -1.0) and math.isclose(float(a[-1]), -math.exp(3.0),
                                                            rel_tol=1e-6)
    assert "delta_bias" in x and x["delta_bias"].shape == (64,)
    bias = torch.nn.functional.softplus(x["delta_bias"].double())
    assert float(bias.min()) >= 1e-3 * 0.999 and float(bias.max()) <= 1e-1 * 1.001
    wl = synth.workload("long", L=16, Dn=64)
    xl = synth.scan_inputs(wl)
    assert "delta_bias" not in xl
    d = xl["delta"].float()
    assert float(d.min()) >= 1e-3 * 0.99 and float(d.max()) <= 1e-1 * 1.01
    assert math.isclose(float(xl["A"][0, -1]), -math.exp(4.0), rel_tol=1e-6)


def test_algorithmic_bytes_matches_shapes():
    w = synth.workload("m130m")
    assert synth.algorithmic_bytes(w) == 202_485_760
    assert synth.algorithmic_bytes(synth.workload("m3b")) == 1_344_643_072
