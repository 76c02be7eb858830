"""GPU parity of ms_scan_fwd_dtproj (the scan with the low-rank step
projection fused in) against the fp64 oracle's scan_dtproj, through the C
ABI, on the same seeded inputs.  Bounds as for the plain scan: fp32 io
1e-4 (1 + |ref|); bf16 io 2 ulp + 1e-3 against the oracle run on the same
bf16 inputs; h_last 1e-4 (1 + |ref|).  The projection is accumulated in fp32
on the GPU and in fp64 in the oracle; neither rounds it to the io type."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import DISCS, assert_within, disc_kw, sample_channels

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(batch, L, Dn, N, rank, io, seed):
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, N=N, io=io)
    x = synth.scan_inputs(w, device=DEV, seed=seed)
    x.update(synth.dtproj_inputs(w, rank, device=DEV, seed=seed))
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 7)
    x["delta_bias"] = torch.randn(Dn, generator=g, device=DEV) * 0.3
    x["h0"] = torch.randn(batch, Dn, N, generator=g, device=DEV)
    return x


def _run(ms, x, disc, softplus=True, optional=True):
    kw = disc_kw(disc)
    h_last = torch.full_like(x["h0"], float("nan"))
    opt = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], h0=x["h0"]) if optional else {}
    y = ms.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"],
                           softplus=softplus, h_last=h_last, **opt, **kw)
    torch.cuda.synchronize()
    ref_y, ref_h = oracle.scan_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"],
                                      softplus=softplus, **opt, **kw)
    return y, h_last, ref_y, ref_h


SHAPES = [
    # batch, L, d_inner, d_state, rank, io
    (1, 1, 64, 16, 16, "f32"),       # one step
    (2, 37, 70, 16, 5, "f32"),       # ragged L, tail tile, rank not a multiple of 4
    (1, 300, 130, 8, 48, "bf16"),    # two K slices, tail tile
    (2, 257, 64, 16, 64, "bf16"),    # the largest rank
    (1, 1009, 96, 16, 1, "bf16"),    # rank 1, several segments, ragged end
    (3, 40, 33, 8, 33, "f32"),       # rank 33: a one-column second slice
    (2, 2100, 192, 16, 16, "bf16"),  # many segments
    # the row kernel (d_state 9..16, d_inner a multiple of 8 / 4): the delta
    # tile formed on the matrix cores by one wave of each workgroup
    (2, 300, 96, 12, 16, "bf16"),    # padded states
    (1, 500, 64, 9, 33, "f32"),      # rank 33: element loads, one-column second slice
    (2, 1100, 128, 13, 48, "bf16"),  # a cut sequence: summary and main with the projection
    (2, 200, 64, 16, 20, "bf16"),    # rank not a multiple of 8: element loads
    (1, 77, 4104, 16, 64, "bf16"),   # a channel tail inside the last workgroup
    # row kernels with 2 or 4 rows per channel (d_state 17..128, batch x
    # d_inner filling the chip uncut): the 16-channel delta tile is formed
    # whole and the workgroup's 8 or 4 channels read from it
    (2, 70, 2048, 32, 16, "bf16"),   # 2 rows per channel
    (1, 45, 2052, 48, 33, "f32"),    # 4 rows, padded states, element loads of x and W
    (1, 20, 4100, 24, 16, "f32"),    # 2 rows, a channel tail inside the last workgroup
    (1, 40, 2048, 100, 64, "bf16"),  # 4 rows x 2 states per lane, padded
    (2, 33, 1024, 128, 20, "bf16"),  # 4 rows x 2 states per lane, rank not a multiple of 8
]


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}L{}D{}N{}R{}{}".format(*s))
def test_dtproj_shapes(gpu, shape, disc):
    batch, L, Dn, N, rank, io = shape
    x = _inputs(batch, L, Dn, N, rank, io, seed=61)
    y, hl, ry, rh = _run(gpu, x, disc)
    assert_within(y, ry, io, "y")
    assert_within(hl, rh, "f32", "h_last")


def test_dtproj_without_optional_terms(gpu):
    x = _inputs(2, 150, 64, 16, 16, "bf16", seed=62)
    y, hl, ry, rh = _run(gpu, x, "euler", optional=False)
    assert_within(y, ry, "bf16", "y")
    assert_within(hl, rh, "f32", "h_last")


def test_dtproj_softplus_off(gpu):
    x = _inputs(1, 200, 64, 16, 8, "f32", seed=63)
    # keep the linear step positive and small without the softplus
    x["dt_low"] = x["dt_low"].abs() * 0.05
    x["W_dt"] = x["W_dt"].abs()
    x["delta_bias"] = x["delta_bias"].abs() * 0.01
    y, hl, ry, rh = _run(gpu, x, "zoh", softplus=False)
    assert_within(y, ry, "f32", "y")
    assert_within(hl, rh, "f32", "h_last")


def test_dtproj_deterministic(gpu):
    x = _inputs(2, 1000, 192, 16, 16, "bf16", seed=64)
    y1 = gpu.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"], D=x["D"],
                             z=x["z"], delta_bias=x["delta_bias"])
    y2 = gpu.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"], D=x["D"],
                             z=x["z"], delta_bias=x["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_dtproj_130m_layer_full(gpu):
    """The 130M-layer workload (B8 L2048 D1536 N16, bf16) with a rank-16 step
    projection, in the launch configuration the benchmark times; every output
    against the oracle."""
    w = synth.workload("m130m")
    x = synth.scan_inputs(w, device=DEV, seed=0)
    x.update(synth.dtproj_inputs(w, 16, device=DEV, seed=0))
    y = gpu.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"], D=x["D"],
                            z=x["z"], delta_bias=x.get("delta_bias"))
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    idx = np.arange(w.Dn)  # every channel
    ii = torch.as_tensor(idx, device=DEV)
    b = x.get("delta_bias")
    ry, _ = oracle.scan_dtproj(x["u"].index_select(2, ii), x["dt_low"],
                               x["W_dt"].index_select(0, ii), x["A"].index_select(0, ii),
                               x["B"], x["C"], D=x["D"].index_select(0, ii),
                               z=x["z"].index_select(2, ii),
                               delta_bias=b.index_select(0, ii) if b is not None else None,
                               softplus=w.softplus)
    assert_within(y.index_select(2, ii), ry, "bf16", "y")


@pytest.mark.parametrize("name,disc,rank", [("wide128", "euler", 48), ("wide64", "euler", 48),
                                            ("wide64", "zoh", 16)],
                         ids=["wide128-euler", "wide64-euler", "wide64-zoh"])
def test_dtproj_wide_workloads_sampled(gpu, name, disc, rank):
    """The wide-state workloads (B2 L8192 D1536, d_state 128 or 64, bf16) with
    the step projection fused, on the row kernels with 4 rows per channel;
    96 sampled channels against the oracle."""
    w = synth.workload(name)
    x = synth.scan_inputs(w, device=DEV, seed=0)
    x.update(synth.dtproj_inputs(w, rank, device=DEV, seed=0))
    y = gpu.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"], D=x["D"],
                            z=x["z"], delta_bias=x.get("delta_bias"), softplus=w.softplus,
                            **disc_kw(disc))
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    ii = torch.as_tensor(sample_channels(w.Dn, 96, seed=3), device=DEV)
    b = x.get("delta_bias")
    ry, _ = oracle.scan_dtproj(x["u"].index_select(2, ii), x["dt_low"],
                               x["W_dt"].index_select(0, ii), x["A"].index_select(0, ii),
                               x["B"], x["C"], D=x["D"].index_select(0, ii),
                               z=x["z"].index_select(2, ii),
                               delta_bias=b.index_select(0, ii) if b is not None else None,
                               softplus=w.softplus, **disc_kw(disc))
    assert_within(y.index_select(2, ii), ry, "bf16", "y")
    del x, y
    torch.cuda.empty_cache()
