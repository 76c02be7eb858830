"""More than 2^31 elements in one call (B1, L = 2^21 + 37, d_inner 1024:
2,147,521,536 elements, 4.3 GB per bf16 tensor), so that any element index or
byte offset kept in 32 bits would wrap in the last 37 timesteps.  The scan at
d_state 16 takes the row kernel with the sequence cut into segments (1024
channels alone give too few waves), so the segment starts, the carry pass and
h_last are exercised at these offsets too.  Sampled channels (both ends, tile
edges, random picks) are compared over the whole sequence with the fp64
oracle on the same inputs; channels are independent, so the oracle on a
subset is exact there."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, oracle_on_channels, sample_channels

pytestmark = pytest.mark.gpu
DEV = "cuda"
L_HUGE = (1 << 21) + 37
DN_HUGE = 1024


def test_scan_past_2_31_elements(gpu):
    w = synth.workload("m130m", batch=1, L=L_HUGE, Dn=DN_HUGE)
    assert w.batch * w.L * w.Dn > 2**31
    x = synth.scan_inputs(w, device=DEV, seed=97)
    hl = torch.empty(w.batch, w.Dn, w.N, device=DEV)
    y = gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                     delta_bias=x.get("delta_bias"), softplus=w.softplus, h_last=hl)
    torch.cuda.synchronize()
    idx = sample_channels(w.Dn, 24, seed=8)
    yr, hr = oracle_on_channels(x, idx, w.softplus, False)
    ii = torch.as_tensor(idx, device=DEV)
    assert_within(y.index_select(2, ii), yr, "bf16")
    assert_within(hl.index_select(1, ii), hr, "f32", "h_last")
    # the rows past element 2^31 of the whole tensor are finite everywhere
    assert torch.isfinite(y[:, -64:, :].float()).all()


def test_conv_past_2_31_elements(gpu):
    w = synth.workload("m130m", batch=1, L=L_HUGE, Dn=DN_HUGE)
    c = synth.conv_inputs(w, 4, device=DEV, seed=98)
    u = gpu.conv1d_silu(c["x"], c["weight"], c["bias"])
    torch.cuda.synchronize()
    idx = sample_channels(w.Dn, 16, seed=9)
    ii = torch.as_tensor(idx, device=DEV)
    ref = oracle.conv1d(c["x"].index_select(2, ii), c["weight"].index_select(0, ii),
                        c["bias"].index_select(0, ii))
    assert_within(u.index_select(2, ii), ref, "bf16")


def test_decode_past_2_31_states(gpu):
    """A decode state of more than 2^31 values (batch 4096 x d_inner 32768 x
    d_state 16 + one batch row: 8.6 GB of fp32 h), two steps; sampled channels
    of every batch row against the oracle's own fp64 state."""
    w = synth.workload("decode", batch=4097, Dn=32768, steps=2)
    assert w.batch * w.Dn * w.N > 2**31
    x = synth.decode_inputs(w, device=DEV, seed=99)
    h = x["h0"].clone()
    idx = sample_channels(w.Dn, 8, seed=10)
    ii = torch.as_tensor(idx, device=DEV)
    href = x["h0"].index_select(1, ii).double().cpu().numpy()
    b = x.get("delta_bias")
    for t in range(w.steps):
        y = gpu.state_update(h, x["x"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t],
                             D=x["D"], z_t=x["z"][t], delta_bias=b, softplus=w.softplus)
        torch.cuda.synchronize()
        yr, href = oracle.step(href, x["x"][t].index_select(1, ii), x["delta"][t].index_select(1, ii),
                               x["A"].index_select(0, ii), x["B"][t], x["C"][t],
                               D=x["D"].index_select(0, ii), z=x["z"][t].index_select(1, ii),
                               delta_bias=b.index_select(0, ii) if b is not None else None,
                               softplus=w.softplus)
        assert_within(y.index_select(1, ii), yr, "bf16", f"y step {t}")
        assert_within(h.index_select(1, ii), href, "f32", f"h step {t}")
