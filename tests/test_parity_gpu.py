"""GPU parity: ms_scan_fwd (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, within the stated tolerances.

Small cases compare every output; the full-size layer shapes compare sampled
channels over the whole sequence (channels are independent, so the oracle on a
channel subset is exactly the oracle's value there), in the same launch
configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import DISCS, assert_within, disc_kw, oracle_on_channels, sample_channels

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _kw(zoh):
    """zoh: a bool (Euler / ZOH) or a discretisation name."""
    return disc_kw(zoh) if isinstance(zoh, str) else {"zoh": bool(zoh)}


def _run(ms, x, softplus, zoh, **kw):
    y = ms.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x.get("D"), z=x.get("z"),
                    delta_bias=x.get("delta_bias"), softplus=softplus, **_kw(zoh), **kw)
    torch.cuda.synchronize()
    return y


def _oracle_full(x, softplus, zoh, h0=None):
    return oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x.get("D"), z=x.get("z"),
                       delta_bias=x.get("delta_bias"), h0=h0, softplus=softplus, **_kw(zoh))


@pytest.mark.parametrize("zoh", DISCS)
def test_tiny_workload_full(gpu, zoh):
    w = synth.workload("tiny")
    x = synth.scan_inputs(w, device=DEV, seed=0)
    h_last = torch.empty(w.batch, w.Dn, w.N, device=DEV)
    y = _run(gpu, x, True, zoh, h_last=h_last)
    yr, hr = _oracle_full(x, True, zoh)
    assert_within(y, yr, "f32")
    assert_within(h_last, hr, "f32", "h_last")


EDGE = [
    # batch, L, Dn, N, io
    (1, 1, 64, 16, "f32"),
    (1, 2, 1, 16, "f32"),
    (2, 1009, 70, 16, "bf16"),
    (3, 4099, 130, 8, "f32"),
    (1, 777, 33, 1, "f32"),
    (2, 300, 65, 3, "bf16"),
    (1, 520, 64, 17, "f32"),
    (1, 400, 96, 32, "bf16"),
    (1, 333, 64, 33, "f32"),
    (2, 2500, 64, 64, "bf16"),
    (1, 260, 40, 100, "f32"),
    (2, 300, 70, 80, "bf16"),   # bf16 rows padded to the 128-state tile
    (1, 350, 64, 40, "bf16"),   # bf16, padded to 64 states (lane or tile)
    (1, 1100, 128, 128, "bf16"),
    # row kernels (d_state 9..16): padded states, channel tails inside a
    # 16-channel workgroup, and sequences cut into several segments
    (1, 2000, 48, 12, "bf16"),
    (2, 777, 20, 9, "f32"),
    (1, 300, 17, 15, "f32"),
    (3, 5000, 33, 16, "bf16"),
    (1, 16, 16, 16, "f32"),
    (1, 17, 5, 13, "bf16"),
    # row kernels with 2 or 4 rows per channel (d_state 17..64) and 2 states
    # per lane (65..128): taken when batch x d_inner fills the chip uncut
    # (2048 waves); padded states, and a channel tail inside the last
    # 8-channel workgroup (fp32, 2 rows)
    (2, 300, 2048, 32, "bf16"),
    (2, 277, 2048, 20, "f32"),
    (1, 250, 2048, 64, "bf16"),
    (1, 190, 2056, 50, "bf16"),
    (2, 190, 2052, 30, "f32"),
    (1, 200, 2048, 128, "f32"),
    (1, 150, 2048, 100, "bf16"),
    # d_state 33..64 with Euler: rows once batch x d_inner >= 8192 (the lane
    # kernel below that); padded states and a channel tail
    (4, 100, 2048, 48, "bf16"),
    (2, 70, 4100, 64, "f32"),
]


@pytest.mark.parametrize("zoh", DISCS)
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "B{}L{}D{}N{}{}".format(*s))
def test_edge_shapes(gpu, shape, zoh):
    batch, L, Dn, N, io = shape
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, N=N, io=io)
    x = synth.scan_inputs(w, device=DEV, seed=11)
    h_last = torch.empty(batch, Dn, N, device=DEV)
    y = _run(gpu, x, True, zoh, h_last=h_last)
    yr, hr = _oracle_full(x, True, zoh)
    assert_within(y, yr, io)
    assert_within(h_last, hr, "f32", "h_last")


@pytest.mark.parametrize("variant", ["no_z", "no_D", "no_bias", "softplus_off", "none"])
def test_optional_terms(gpu, variant):
    w = synth.workload("m130m", batch=2, L=700, Dn=96)
    x = synth.scan_inputs(w, device=DEV, seed=5)
    softplus = True
    if variant in ("no_z", "none"):
        x["z"] = None
    if variant in ("no_D", "none"):
        x["D"] = None
    if variant in ("no_bias", "none"):
        x["delta_bias"] = None
    if variant == "softplus_off":
        # positive steps drawn directly, no softplus and no bias
        x["delta"] = (torch.rand(x["delta"].shape, device=DEV) * 0.1 + 1e-3).to(torch.bfloat16)
        x["delta_bias"] = None
        softplus = False
    y = _run(gpu, x, softplus, False)
    yr, _ = _oracle_full(x, softplus, False)
    assert_within(y, yr, "bf16")


def test_zero_bias_equals_null_bias(gpu):
    w = synth.workload("tiny", L=300)
    x = synth.scan_inputs(w, device=DEV, seed=2)
    assert torch.count_nonzero(x["delta_bias"]) == 0
    y0 = _run(gpu, x, True, False).clone()
    x2 = dict(x)
    x2["delta_bias"] = None
    y1 = _run(gpu, x2, True, False)
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("zoh", DISCS)
def test_special_cases_zero_A_and_zero_step(gpu, zoh):
    w = synth.workload("tiny", batch=2, L=513, Dn=80, N=16)
    x = synth.scan_inputs(w, device=DEV, seed=3)
    xa = dict(x)
    xa["A"] = torch.zeros_like(x["A"])          # prefix-sum regime
    y = _run(gpu, xa, True, zoh)
    yr, _ = _oracle_full(xa, True, zoh)
    assert_within(y, yr, "f32")
    xd = dict(x)
    xd["delta"] = torch.zeros_like(x["delta"])  # dt = 0: state frozen at h0
    xd["delta_bias"] = None
    h0 = torch.randn(2, 80, 16, device=DEV)
    hl = torch.empty_like(h0)
    y = _run(gpu, xd, False, zoh, h0=h0, h_last=hl)
    yr, hr = _oracle_full(xd, False, zoh, h0=h0)
    assert_within(y, yr, "f32")
    assert torch.equal(hl, h0)


def test_split_resume_matches_single_scan(gpu):
    w = synth.workload("m130m", batch=2, L=3000, Dn=128)
    x = synth.scan_inputs(w, device=DEV, seed=4)
    h0 = torch.randn(2, 128, 16, device=DEV) * 0.1
    hl = torch.empty_like(h0)
    y = _run(gpu, x, True, False, h0=h0, h_last=hl)
    yr, hr = _oracle_full(x, True, False, h0=h0)
    assert_within(y, yr, "bf16")
    assert_within(hl, hr, "f32", "h_last")
    L1 = 1234
    first = {k: (v[:, :L1].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in x.items()}
    second = {k: (v[:, L1:].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
              for k, v in x.items()}
    hm = torch.empty_like(h0)
    y1 = _run(gpu, first, True, False, h0=h0, h_last=hm)
    h2 = torch.empty_like(h0)
    y2 = _run(gpu, second, True, False, h0=hm, h_last=h2)
    assert_within(torch.cat([y1, y2], dim=1), yr, "bf16", "split y")
    assert_within(h2, hr, "f32", "split h_last")
    # h0 may alias h_last
    hh = h0.clone()
    y3 = _run(gpu, x, True, False, h0=hh, h_last=hh)
    assert torch.equal(y3, y)
    assert torch.equal(hh, hl)


# h_last may alias h0 (include/msscan.h).  With one segment each channel's
# lanes read h0 before they write h_last; with several, the first segment
# starts from the carry pass's copy of h0.  Cases: the full 3B layer (row
# kernels, one segment), and segmented plans of the row, lane and tile kernels.
# The last two cut the sequence into 2049 segments of 64 steps (one wave per
# segment), so their carries take the split form for chains of 1024 or more
# segments, with h0 as the initial state (the bilinear one with products of
# A_bar as decays).
ALIAS = [("m3b", None, "euler"), ("tiny", (1, 6000, 40, 16), "zoh"),
         ("tiny", (2, 3000, 64, 32), "euler"), ("tiny", (1, 3000, 64, 64), "zoh"),
         ("tiny", (1, 4000, 64, 8), "bilinear"), ("tiny", (1, 300, 2048, 128), "bilinear"),
         ("tiny", (1, 131077, 64, 8), "euler"), ("tiny", (1, 131077, 64, 8), "bilinear")]


@pytest.mark.parametrize("name,shape,disc", ALIAS,
                         ids=["m3b", "rows-seg", "lane32-seg", "tile64-seg", "lane8-seg",
                              "rows128", "lane8-long-chain", "lane8-long-chain-bil"])
def test_h0_aliases_h_last(gpu, name, shape, disc):
    if shape is None:
        w = synth.workload(name)
    else:
        b, L, Dn, N = shape
        w = synth.workload(name, batch=b, L=L, Dn=Dn, N=N, io="bf16")
    x = synth.scan_inputs(w, device=DEV, seed=12)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    h0 = torch.randn(w.batch, w.Dn, w.N, generator=g, device=DEV) * 0.5
    hl = torch.empty_like(h0)
    y = _run(gpu, x, w.softplus, disc, h0=h0, h_last=hl).clone()
    hh = h0.clone()
    y2 = _run(gpu, x, w.softplus, disc, h0=hh, h_last=hh)
    assert torch.equal(y2, y)
    assert torch.equal(hh, hl)
    if shape is not None:
        yr, hr = _oracle_full(x, w.softplus, disc, h0=h0)
        assert_within(y, yr, "bf16")
        assert_within(hl, hr, "f32", "h_last")
    del x, y, y2
    torch.cuda.empty_cache()


def test_deterministic_and_workspace_reuse(gpu):
    w = synth.workload("m130m", batch=3, L=4096, Dn=192)
    x = synth.scan_inputs(w, device=DEV, seed=6)
    n = gpu.workspace_bytes(3, 4096, 192, 16, gpu.MS_BF16)
    assert n > 0
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN-filled scratch
    y1 = _run(gpu, x, True, False, workspace=ws).clone()
    y2 = _run(gpu, x, True, False, workspace=ws)
    assert torch.equal(y1, y2)


def test_outputs_stay_in_bounds(gpu):
    """Tail channels and the last chunk must not write past y or h_last."""
    batch, L, Dn, N = 2, 1500, 70, 16
    w = synth.workload("m130m", batch=batch, L=L, Dn=Dn)
    x = synth.scan_inputs(w, device=DEV, seed=7)
    pad = 4096
    ybuf = torch.full((batch * L * Dn + pad,), 12345.0, device=DEV).to(torch.bfloat16)
    hbuf = torch.full((batch * Dn * N + pad,), 777.0, device=DEV)
    y = ybuf[: batch * L * Dn].view(batch, L, Dn)
    hl = hbuf[: batch * Dn * N].view(batch, Dn, N)
    _run(gpu, x, True, False, y=y, h_last=hl)
    assert torch.all(ybuf[batch * L * Dn:].float() == 12352.0)  # bf16(12345) = 12352
    assert torch.all(hbuf[batch * Dn * N:] == 777.0)


def test_nan_stays_in_its_channel(gpu):
    w = synth.workload("m130m", batch=2, L=1024, Dn=128)
    x = synth.scan_inputs(w, device=DEV, seed=8)
    b0, t0, d0 = 1, 500, 77
    x["u"][b0, t0, d0] = float("nan")
    y = _run(gpu, x, True, False).float().cpu()
    bad = torch.isnan(y)
    assert bad[b0, t0:, d0].all()
    bad[b0, t0:, d0] = False
    assert not bad.any()


# ---------------------------------------------------------------- full sizes ---
# k = 0: every channel (the oracle runs at ~1e8 elements/s on the host: about a
# second for the 130M layer, a few for the 3B layer)
@pytest.mark.parametrize("name,zoh,k", [("m130m", "euler", 0), ("m3b", "euler", 0),
                                         ("m3b", "zoh", 0), ("m3b", "bilinear", 0),
                                         ("wide128", "euler", 96), ("wide64", "zoh", 96)],
                         ids=["m130m-euler", "m3b-euler", "m3b-zoh", "m3b-bilinear",
                              "wide128-euler", "wide64-zoh"])
def test_layer_workloads_full(gpu, name, zoh, k):
    w = synth.workload(name)
    x = synth.scan_inputs(w, device=DEV, seed=0)
    y = _run(gpu, x, w.softplus, zoh)
    idx = sample_channels(w.Dn, k, seed=1) if k else np.arange(w.Dn)
    yr, _ = oracle_on_channels(x, idx, w.softplus, **_kw(zoh))
    got = y.index_select(2, torch.as_tensor(idx, device=DEV))
    assert_within(got, yr, w.io)
    # Whole-tensor properties at full size: finite, and not all zero.
    assert torch.isfinite(y.float()).all()
    del x, y
    torch.cuda.empty_cache()


def test_long_context_sampled(gpu):
    w = synth.workload("long")
    x = synth.scan_inputs(w, device=DEV, seed=0)
    hl = torch.empty(w.batch, w.Dn, w.N, device=DEV)
    y = _run(gpu, x, w.softplus, False, h_last=hl)
    idx = sample_channels(w.Dn, 48, seed=2)
    yr, hr = oracle_on_channels(x, idx, w.softplus, False)
    ii = torch.as_tensor(idx, device=DEV)
    assert_within(y.index_select(2, ii), yr, w.io)
    assert_within(hl.index_select(1, ii), hr, "f32", "h_last")
    assert torch.isfinite(y.float()).all()
    del x, y
    torch.cuda.empty_cache()
