"""GPU parity of ms_scan_bwd (gradients of the scan) against the fp64 oracle's
backward (itself pinned to finite differences of the forward oracle), through
the C ABI, on the same seeded inputs.

Bound.  Several gradients are sums of many terms of both signs (dA, dD and
dbias over batch and time; dB and dC over channels), so their fp32 rounding
scales with the size of the terms, not of the sum.  Every gradient tensor g is
therefore checked as |g_gpu - g_ref| <= rtol * (|g_ref| + rms(g_ref)), with
rtol = 2e-4 for fp32 io and, for the bf16 io outputs du / ddelta / dz, the
bf16 rounding of the stored value added (2 bf16 ulp).  A wrong term or index
gives O(1) relative errors and fails it."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import DISCS, disc_kw

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(got, ref, io, what, rtol=2e-4):
    got = got.detach().to("cpu").double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    lim = rtol * (np.abs(ref) + rms) + 1e-30
    if io == "bf16":
        a = np.abs(ref)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        lim = lim + 2.0 * np.where(a > 0, np.exp2(e - 7.0), 0.0)
    err = np.abs(got - ref)
    bad = ~(err <= lim)
    if bad.any():
        i = np.argwhere(bad)[:4].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside bound; worst "
                             f"err/lim {float(np.max(err / lim)):.3g}; at {i} got "
                             f"{[float(got[tuple(k)]) for k in i]} ref "
                             f"{[float(ref[tuple(k)]) for k in i]}")


def _inputs(batch, L, Dn, N, io, seed, optional=True):
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, N=N, io=io)
    x = synth.scan_inputs(w, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1000)
    x["dy"] = torch.randn(batch, L, Dn, generator=g, device=DEV).to(x["u"].dtype)
    if optional:
        x["h0"] = torch.randn(batch, Dn, N, generator=g, device=DEV)
        x["dh_last"] = torch.randn(batch, Dn, N, generator=g, device=DEV)
        x["delta_bias"] = torch.randn(Dn, generator=g, device=DEV) * 0.3
    else:
        x["z"] = None
        x["D"] = None
        x["delta_bias"] = None
    return x


def _compare(ms, x, io, disc, softplus=True):
    kw = disc_kw(disc)
    got = ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x.get("D"),
                      z=x.get("z"), delta_bias=x.get("delta_bias"), softplus=softplus,
                      h0=x.get("h0"), dh_last=x.get("dh_last"), **kw)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x.get("D"),
                          z=x.get("z"), delta_bias=x.get("delta_bias"), h0=x.get("h0"),
                          dh_last=x.get("dh_last"), softplus=softplus, **kw)
    for k in ("du", "ddelta", "dz"):
        if ref[k] is not None:
            _check(got[k], ref[k], io, k)
    for k in ("dA", "dB", "dC", "dD", "dbias", "dh0"):
        if ref[k] is not None:
            _check(got[k], ref[k], "f32", k)


SHAPES = [
    # batch, L, Dn, N, io
    (1, 1, 4, 4, "f32"),
    (2, 37, 70, 16, "f32"),    # L not a multiple of the segment, a tail tile
    (1, 100, 64, 8, "bf16"),
    (2, 257, 130, 16, "bf16"),
    (1, 48, 33, 5, "f32"),     # d_state 5: masked states
    (2, 90, 70, 12, "bf16"),   # d_state 12 with bf16 io: staged B/C rows padded to 16
    (3, 16, 64, 1, "f32"),
]

# Shapes with at least 512 16-channel tiles over the batch and d_state 9..16
# take the row-layout backward (a checkpointing forward walk and one reverse
# walk per tile): ragged last blocks, padded states, a channel tail inside the
# last tile (d_inner 4104).
ROWS = [
    (4, 300, 2048, 16, "bf16"),
    (2, 129, 4096, 12, "f32"),
    (1, 77, 8192, 9, "bf16"),
    (2, 20, 4104, 16, "bf16"),
]


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("shape", ROWS, ids=lambda s: "B{}L{}D{}N{}{}".format(*s))
def test_bwd_rows(gpu, shape, disc):
    batch, L, Dn, N, io = shape
    x = _inputs(batch, L, Dn, N, io, seed=41)
    _compare(gpu, x, io, disc)


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "raw_step"])
@pytest.mark.parametrize("disc", DISCS)
def test_bwd_rows_options_off(gpu, disc, softplus):
    """Row-layout backward with no gate, D, bias, h0 or dh_last."""
    x = _inputs(4, 70, 2048, 16, "bf16", seed=42, optional=False)
    if not softplus:
        x["delta"] = (x["delta"].float().abs() * 0.05 + 0.01).to(x["delta"].dtype)
    _compare(gpu, x, "bf16", disc, softplus=softplus)


def test_bwd_rows_deterministic(gpu):
    x = _inputs(4, 200, 2048, 16, "bf16", seed=43)
    g1 = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=x["h0"], dh_last=x["dh_last"])
    g2 = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=x["h0"], dh_last=x["dh_last"])
    torch.cuda.synchronize()
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}L{}D{}N{}{}".format(*s))
def test_bwd_shapes(gpu, shape, disc):
    batch, L, Dn, N, io = shape
    x = _inputs(batch, L, Dn, N, io, seed=31)
    _compare(gpu, x, io, disc)


@pytest.mark.parametrize("disc", DISCS)
def test_bwd_without_optional_terms(gpu, disc):
    x = _inputs(2, 70, 64, 16, "f32", seed=32, optional=False)
    _compare(gpu, x, "f32", disc)


def test_bwd_softplus_off(gpu):
    x = _inputs(1, 90, 64, 16, "f32", seed=33)
    x["delta"] = x["delta"].abs() * 0.05 + 0.01
    x["delta_bias"] = x["delta_bias"].abs() * 0.01
    _compare(gpu, x, "f32", "euler", softplus=False)


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "raw_step"])
@pytest.mark.parametrize("disc", DISCS)
def test_bwd_bf16_options_off(gpu, disc, softplus):
    """bf16 io (inputs staged in LDS; no z reads a zero-size buffer) with no
    gate, D or bias, softplus on and off; L = 70 leaves a partial last
    segment, whose adjoint walk also forms its decay."""
    x = _inputs(2, 70, 64, 16, "bf16", seed=35, optional=False)
    if not softplus:
        x["delta"] = (x["delta"].float().abs() * 0.05 + 0.01).to(x["delta"].dtype)
    _compare(gpu, x, "bf16", disc, softplus=softplus)


def test_bwd_deterministic(gpu):
    x = _inputs(2, 300, 192, 16, "bf16", seed=34)
    g1 = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=x["h0"])
    g2 = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], h0=x["h0"])
    torch.cuda.synchronize()
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k


@pytest.mark.parametrize("disc", DISCS)
def test_bwd_130m_layer(gpu, disc):
    """The 130M-layer shape (B8 L2048 D1536 N16, bf16), every gradient."""
    w = synth.workload("m130m")
    x = synth.scan_inputs(w, device=DEV, seed=0)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    x["dy"] = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV).to(x["u"].dtype)
    _compare(gpu, x, "bf16", disc)


@pytest.mark.parametrize("disc", DISCS)
def test_bwd_zero_A_entries(gpu, disc):
    """Some A entries exactly 0 (and some tiny): the ZOH factor and its
    derivative take their series branch there; every gradient must still
    match the oracle (whose A = 0 case is pinned by finite differences)."""
    x = _inputs(2, 90, 64, 16, "f32", seed=35)
    A = x["A"].clone()
    A[:, 0] = 0.0
    A[::3, 5] = -1e-6
    x["A"] = A
    _compare(gpu, x, "f32", disc)


# ---- d_state 17..128: the state differentiated in slices of 16 ---------------------
WIDE = [
    # batch, L, Dn, N, io
    (1, 40, 24, 32, "f32"),
    (2, 70, 40, 64, "bf16"),
    (1, 33, 17, 24, "f32"),    # last slice half padded
    (1, 50, 16, 100, "bf16"),  # 7 slices, the last with 4 states
    (1, 20, 8, 128, "f32"),
    (1, 1, 64, 48, "f32"),     # a single timestep
    (1, 40, 8192, 32, "bf16"), # 512 16-channel tiles: row-layout slices, y_pre from a forward
]


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "B{}L{}D{}N{}{}".format(*s))
def test_bwd_wide_state(gpu, shape, disc):
    batch, L, Dn, N, io = shape
    x = _inputs(batch, L, Dn, N, io, seed=41)
    _compare(gpu, x, io, disc)


@pytest.mark.parametrize("disc", DISCS)
def test_bwd_wide_without_optional_terms(gpu, disc):
    x = _inputs(2, 60, 48, 32, "bf16", seed=42, optional=False)
    _compare(gpu, x, "bf16", disc)


def test_bwd_wide_deterministic(gpu):
    x = _inputs(2, 200, 96, 64, "bf16", seed=43)
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"])
    kw = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"], dh_last=x["dh_last"])
    g1 = gpu.scan_bwd(*args, **kw)
    g2 = gpu.scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k


def test_bwd_wide_full_channels(gpu):
    """d_state 64 over all 1536 channels of the long-context layer, 4096
    steps (every gradient, dB and dC summed over every channel)."""
    w = synth.workload("long", L=4096)
    x = synth.scan_inputs(w, device=DEV, seed=5)
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    x["dy"] = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV).to(x["u"].dtype)
    _compare(gpu, x, w.io, "euler", softplus=w.softplus)


def _channels(x, idx):
    """The sub-problem made of the channels idx (each channel's recurrence
    is independent; B and C are shared)."""
    ii = torch.as_tensor(idx, device=DEV)
    sub = dict(x)
    for k in ("u", "delta", "z", "dy"):
        if x.get(k) is not None:
            sub[k] = x[k].index_select(2, ii).contiguous()
    for k in ("A", "D", "delta_bias"):
        if x.get(k) is not None:
            sub[k] = x[k].index_select(0, ii).contiguous()
    return sub


def test_bwd_wide_long_context_sampled(gpu):
    """The long-context shape B1 L65536 D1536 N64 (bf16, Euler): the full
    backward's per-channel gradients (du, ddelta, dz, dA, dD, dbias, dh0) on
    48 sampled channels against the oracle run on those channels; and the
    channel sums dB, dC of the sub-problem made of the sampled channels
    (through the same kernels) against the oracle's."""
    from helpers import sample_channels
    w = synth.workload("long", L=65536)
    x = synth.scan_inputs(w, device=DEV, seed=6)
    g = torch.Generator(device=DEV)
    g.manual_seed(79)
    x["dy"] = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV).to(x["u"].dtype)
    idx = sample_channels(w.Dn, 48, seed=3)
    full = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                        delta_bias=x.get("delta_bias"), softplus=w.softplus)
    torch.cuda.synchronize()
    sub = _channels(x, idx)
    ref = oracle.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dy"],
                          D=sub["D"], z=sub["z"], delta_bias=sub.get("delta_bias"),
                          softplus=w.softplus)
    ii = torch.as_tensor(idx, device=DEV)
    for k in ("du", "ddelta", "dz"):
        _check(full[k].index_select(2, ii), ref[k], w.io, k)
    _check(full["dA"].index_select(0, ii), ref["dA"], "f32", "dA")
    _check(full["dD"].index_select(0, ii), ref["dD"], "f32", "dD")
    part = gpu.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dy"],
                        D=sub["D"], z=sub["z"], delta_bias=sub.get("delta_bias"),
                        softplus=w.softplus)
    torch.cuda.synchronize()
    _check(part["dB"], ref["dB"], "f32", "dB")
    _check(part["dC"], ref["dC"], "f32", "dC")
    del x, full, part
    torch.cuda.empty_cache()


def test_bwd_past_2_31_elements_sampled(gpu):
    """More than 2^31 elements in one backward call (B1, L = 2^21 + 37,
    d_inner 1024, d_state 16, bf16, Euler, softplus and bias): the per-channel
    gradients on 24 sampled channels against the oracle run on those
    channels, and the channel sums dB, dC of the sub-problem made of those
    channels.  Any element index or byte offset kept in 32 bits would wrap in
    the last 37 timesteps."""
    from helpers import sample_channels
    w = synth.workload("m130m", batch=1, L=(1 << 21) + 37, Dn=1024)
    assert w.batch * w.L * w.Dn > 2**31
    x = synth.scan_inputs(w, device=DEV, seed=12)
    g = torch.Generator(device=DEV)
    g.manual_seed(81)
    x["dy"] = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV).to(x["u"].dtype)
    idx = sample_channels(w.Dn, 24, seed=4)
    full = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x["D"], z=x["z"],
                        delta_bias=x.get("delta_bias"), softplus=w.softplus)
    torch.cuda.synchronize()
    sub = _channels(x, idx)
    ref = oracle.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dy"],
                          D=sub["D"], z=sub["z"], delta_bias=sub.get("delta_bias"),
                          softplus=w.softplus)
    ii = torch.as_tensor(idx, device=DEV)
    for k in ("du", "ddelta", "dz"):
        _check(full[k].index_select(2, ii), ref[k], w.io, k)
    for k in ("dA", "dD", "dbias"):
        _check(full[k].index_select(0, ii), ref[k], "f32", k)
    del full
    torch.cuda.empty_cache()
    part = gpu.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dy"],
                        D=sub["D"], z=sub["z"], delta_bias=sub.get("delta_bias"),
                        softplus=w.softplus)
    torch.cuda.synchronize()
    _check(part["dB"], ref["dB"], "f32", "dB")
    _check(part["dC"], ref["dC"], "f32", "dC")
    del x, part
    torch.cuda.empty_cache()


@pytest.mark.parametrize("disc", DISCS)
def test_bwd_long_chain_of_segments(gpu, disc):
    """A segment-layout backward with 1100 16-step segments (L = 17605, a
    ragged last segment): its two carries take the split form for chains of
    1024 or more segments (runs of slots folded per wave, then re-walked from
    their composed starts), forward with h0 and in reverse with dh_last, and
    with the bilinear form's products of A_bar.  Every gradient of every
    channel against the oracle, and bitwise equal on a second call."""
    x = _inputs(1, 16 * 1100 + 5, 64, 16, "f32", seed=44)
    _compare(gpu, x, "f32", disc)
    kw = disc_kw(disc)
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"])
    opt = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"],
               dh_last=x["dh_last"], **kw)
    g1, g2 = gpu.scan_bwd(*args, **opt), gpu.scan_bwd(*args, **opt)
    torch.cuda.synchronize()
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k
