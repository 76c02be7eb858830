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


def test_profile_times_every_backward_launch(gpu):
    """The backward launches two carries (forward starts, adjoint) and three
    reduction kernels per call (dB | dC, then the parameter sums in two levels:
    32 partial rows here, more than one pass adds): each launch is timed on
    its own."""
    w = synth.workload("m130m", batch=2, L=1024, Dn=128)
    x = synth.scan_inputs(w, device="cuda", seed=4)
    dy = torch.randn(w.batch, w.L, w.Dn, device="cuda").to(x["u"].dtype)
    gpu.profile_begin(3)
    for _ in range(3):
        gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                     delta_bias=x["delta_bias"])
    prof = gpu.profile_end()
    assert prof["calls"] == 3
    assert prof["carry"]["launches"] == 6 and prof["reduce"]["launches"] == 9
    assert prof["summary"]["launches"] == 3 and prof["main"]["launches"] == 3
    for k in ("carry", "reduce", "summary", "main"):
        assert prof[k]["mean_ms"] > 0


def test_profile_times_row_backward_launches(gpu):
    """The row-layout backward (at least 512 16-channel tiles): one
    checkpointing forward walk (summary phase), one reverse walk (main) and
    one reduction launch per call (dB | dC and the parameter sums over the
    batch rows together); no carries."""
    w = synth.workload("m130m", batch=4, L=64, Dn=2048)
    x = synth.scan_inputs(w, device="cuda", seed=4)
    dy = torch.randn(w.batch, w.L, w.Dn, device="cuda").to(x["u"].dtype)
    gpu.profile_begin(3)
    for _ in range(3):
        gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                     delta_bias=x["delta_bias"])
    prof = gpu.profile_end()
    assert prof["calls"] == 3
    assert prof["carry"]["launches"] == 0 and prof["reduce"]["launches"] == 3
    assert prof["summary"]["launches"] == 3 and prof["main"]["launches"] == 3
    for k in ("reduce", "summary", "main"):
        assert prof[k]["mean_ms"] > 0


def test_profile_times_every_wide_backward_launch(gpu):
    """The d_state 17-128 backward runs each 16-state slice as its own
    segment-layout backward (gather, walk, carries, gradient pass, sums,
    accumulate): ~40 timed launches per call at d_state 64, every one of them
    recorded, the same number for each call."""
    w = synth.workload("long", L=512, Dn=256)
    x = synth.scan_inputs(w, device="cuda", seed=5)
    dy = torch.randn(w.batch, w.L, w.Dn, device="cuda").to(x["u"].dtype)

    def launches(calls):
        gpu.profile_begin(calls)
        for _ in range(calls):
            gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                         delta_bias=x.get("delta_bias"), softplus=w.softplus)
        prof = gpu.profile_end()
        assert prof["calls"] == calls
        return {k: v["launches"] for k, v in prof.items() if isinstance(v, dict)}

    one, two = launches(1), launches(2)
    assert sum(one.values()) > 16
    assert all(two[k] == 2 * one[k] for k in one)
    assert one["reduce"] >= 4 and one["main"] >= 4  # at least one of each per slice
