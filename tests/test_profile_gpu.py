"""GPU: the kernel-timing facility (ms_profile_begin / ms_profile_end) counts
the launches each call makes, returns positive times, and leaves results
unchanged."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _scan(ms, x, w):
    return ms.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                       delta_bias=x.get("delta_bias"), softplus=w.softplus)


def test_profile_counts_phases_and_keeps_results(gpu):
    w = synth.workload("m130m", batch=2, L=4096, Dn=256)
    x = synth.scan_inputs(w, device="cuda", seed=3)
    y0 = _scan(gpu, x, w).clone()
    gpu.profile_begin(2)
    ys = [_scan(gpu, x, w) for _ in range(3)]  # the third call is not timed
    prof = gpu.profile_end()
    torch.cuda.synchronize()
    for y in ys:
        assert torch.equal(y, y0)
    assert prof["calls"] == 2
    assert prof["main"]["launches"] == 2
    assert prof["main"]["mean_ms"] > 0
    # this shape is cut into segments: summary and carry passes run once per call
    assert prof["summary"]["launches"] == 2 and prof["carry"]["launches"] == 2
    assert prof["step"]["launches"] == 0


def test_profile_times_decode_step(gpu):
    w = synth.workload("decode", steps=2)
    d = synth.decode_inputs(w, device="cuda", seed=0)
    h = d["h0"].clone()
    gpu.profile_begin(4)
    for t in range(2):
        gpu.state_update(h, d["x"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t], D=d["D"],
                         z_t=d["z"][t], delta_bias=d.get("delta_bias"), softplus=w.softplus)
    prof = gpu.profile_end()
    assert prof["calls"] == 2
    assert prof["step"]["launches"] == 2 and prof["step"]["mean_ms"] > 0
    assert prof["main"]["launches"] == 0
    with pytest.raises(gpu.MsError):
        gpu.profile_end()  # already closed
