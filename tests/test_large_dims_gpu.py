"""Very wide channel counts: d_inner of 200k-300k with a ragged last tile
(thousands of 64-channel tiles in the grid, byte offsets past 2^24), so that
a 32-bit offset or grid-mapping mistake would show.  Sampled channels (both
ends, tile edges, random picks) are compared with the fp64 oracle on the same
inputs; channels are independent, so the oracle on a subset is exact there.
Bounds as in the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, disc_kw, oracle_on_channels, sample_channels

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("disc", ["euler", "zoh"])
def test_scan_wide(gpu, disc):
    w = synth.workload("tiny", batch=2, L=70, Dn=200_003, N=16, io="bf16")
    x = synth.scan_inputs(w, device=DEV, seed=91)
    hl = torch.empty(w.batch, w.Dn, w.N, device=DEV)
    y = gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                     delta_bias=x.get("delta_bias"), h_last=hl, **disc_kw(disc))
    torch.cuda.synchronize()
    idx = sample_channels(w.Dn, 40, seed=5)
    kw = disc_kw(disc)
    yr, hr = oracle_on_channels(x, idx, w.softplus, kw["zoh"], bilinear=kw["bilinear"])
    ii = torch.as_tensor(idx, device=DEV)
    assert_within(y.index_select(2, ii), yr, "bf16")
    assert_within(hl.index_select(1, ii), hr, "f32", "h_last")
    assert torch.isfinite(y.float()).all()


def test_decode_wide(gpu):
    w = synth.workload("decode", batch=3, Dn=300_001, steps=2)
    x = synth.decode_inputs(w, device=DEV, seed=92)
    h = x["h0"].clone()
    idx = sample_channels(w.Dn, 40, seed=6)
    ii = torch.as_tensor(idx, device=DEV)
    href = x["h0"].index_select(1, ii).double().cpu().numpy()
    b = x.get("delta_bias")
    for t in range(w.steps):
        # per-step slices of an odd-sized row are not 16-byte aligned (the
        # library requires it): pass aligned copies
        xt, dt_, zt = x["x"][t].clone(), x["delta"][t].clone(), x["z"][t].clone()
        y = gpu.state_update(h, xt, dt_, x["A"], x["B"][t].clone(), x["C"][t].clone(),
                             D=x["D"], z_t=zt, delta_bias=b)
        torch.cuda.synchronize()
        yr, href = oracle.step(href, x["x"][t].index_select(1, ii), x["delta"][t].index_select(1, ii),
                               x["A"].index_select(0, ii), x["B"][t], x["C"][t],
                               D=x["D"].index_select(0, ii), z=x["z"][t].index_select(1, ii),
                               delta_bias=b.index_select(0, ii) if b is not None else None)
        assert_within(y.index_select(1, ii), yr, "bf16", f"y step {t}")
        assert_within(h.index_select(1, ii), href, "f32", f"h step {t}")


def test_conv_wide(gpu):
    w = synth.workload("tiny", batch=2, L=40, Dn=300_004, N=16, io="bf16")
    c = synth.conv_inputs(w, 4, device=DEV, seed=93, history=True)
    u = gpu.conv1d_silu(c["x"], c["weight"], c["bias"], c["x_prev"])
    torch.cuda.synchronize()
    idx = sample_channels(w.Dn, 40, seed=7)
    ii = torch.as_tensor(idx, device=DEV)
    ref = oracle.conv1d(c["x"].index_select(2, ii), c["weight"].index_select(0, ii),
                        c["bias"].index_select(0, ii), c["x_prev"].index_select(2, ii))
    assert_within(u.index_select(2, ii), ref, "bf16")
