"""GPU parity of ms_state_update (recurrent decode) against the fp64 oracle.

The oracle keeps its own fp64 state across all steps (it is never re-synced
from the GPU), and the GPU's y_t and h are checked after every step.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import DISCS, assert_within, disc_kw

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(ms, h, x, t, softplus, disc):
    # per-step slices are cloned so every base pointer is a fresh (aligned) allocation
    y = ms.state_update(h, x["x"][t].clone(), x["delta"][t].clone(), x["A"], x["B"][t].clone(),
                        x["C"][t].clone(), D=x.get("D"),
                        z_t=x["z"][t].clone() if x.get("z") is not None else None,
                        delta_bias=x.get("delta_bias"), softplus=softplus, **disc_kw(disc))
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("disc", DISCS)
def test_decode_workload_every_step(gpu, disc):
    w = synth.workload("decode")
    x = synth.decode_inputs(w, device=DEV, seed=0)
    h = x["h0"].clone()
    href = x["h0"].double().cpu().numpy()
    A, D, bias = x["A"], x["D"], x.get("delta_bias")
    for t in range(w.steps):
        y = _step(gpu, h, x, t, True, disc)
        yr, href = oracle.step(href, x["x"][t], x["delta"][t], A, x["B"][t], x["C"][t], D=D,
                               z=x["z"][t], delta_bias=bias, softplus=True, **disc_kw(disc))
        assert_within(y, yr, "bf16", f"y step {t}")
        assert_within(h, href, "f32", f"h step {t}")


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 70, 7), (2, 64, 16), (5, 300, 64),
                                   (2, 33, 128), (1, 5, 4), (3, 37, 8), (2, 19, 32),
                                   (1, 3, 12), (2, 70, 100), (1, 40, 17), (2, 65, 24)],
                         ids=lambda s: "B{}D{}N{}".format(*s))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_edge_shapes(gpu, shape, io):
    batch, Dn, N = shape
    w = synth.workload("decode", batch=batch, Dn=Dn, N=N, io=io, steps=5)
    x = synth.decode_inputs(w, device=DEV, seed=3)
    for disc in DISCS:
        h = x["h0"].clone()
        href = x["h0"].double().cpu().numpy()
        for t in range(w.steps):
            y = _step(gpu, h, x, t, True, disc)
            yr, href = oracle.step(href, x["x"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t],
                                   D=x["D"], z=x["z"][t], delta_bias=x.get("delta_bias"),
                                   softplus=True, **disc_kw(disc))
            assert_within(y, yr, io, f"y step {t}")
            assert_within(h, href, "f32", f"h step {t}")


@pytest.mark.parametrize("N", [16, 40, 100])
@pytest.mark.parametrize("disc", DISCS)
def test_steps_equal_scan(gpu, disc, N):
    """L decode steps from h0 reproduce one scan over the same L tokens (at
    d_state 40 and 100 both paths run padded, each in its own way)."""
    batch, L, Dn = 2, 40, 96
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, N=N)
    x = synth.scan_inputs(w, device=DEV, seed=9)
    h0 = torch.randn(batch, Dn, N, device=DEV)
    hl = torch.empty_like(h0)
    ys = gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=h0, h_last=hl, **disc_kw(disc))
    h = h0.clone()
    for t in range(L):
        yt = gpu.state_update(h, x["u"][:, t].contiguous(), x["delta"][:, t].contiguous(),
                              x["A"], x["B"][:, t].contiguous(), x["C"][:, t].contiguous(),
                              D=x["D"], z_t=x["z"][:, t].contiguous(),
                              delta_bias=x["delta_bias"], **disc_kw(disc))
        torch.cuda.synchronize()
        # the two paths round differently; both sit within the fp32 bound of each other
        assert_within(yt, ys[:, t].double().cpu().numpy(), "f32", f"y step {t}")
    assert_within(h, hl.double().cpu().numpy(), "f32", "h")
