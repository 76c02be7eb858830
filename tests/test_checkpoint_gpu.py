"""GPU parity of the checkpointed training pair (ms_scan_fwd_checkpoint and
ms_scan_bwd_checkpoint) through the C ABI, on the seeded inputs of the
backward tests:
  - y and h_last are bit-identical to ms_scan_fwd's (the same kernel
    arithmetic, with the block states stored beside it);
  - checkpoint entry k is h0 at k = 0 and, at the other blocks checked, the
    fp64 oracle's final state after the first 16k steps, to the h_last bound
    1e-4 (1 + |ref|);
  - every gradient against oracle.scan_bwd with the bound of the backward
    tests, and bit-identical to ms_scan_bwd's, which recomputes the same
    states with the same arithmetic."""
import pytest
import torch

import oracle
import synth
from helpers import DISCS, assert_within, disc_kw
from test_bwd_gpu import ROWS, _check, _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRADS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "dbias", "dh0")


def _pair(ms, x, disc, softplus=True):
    kw = disc_kw(disc)
    opt = dict(D=x.get("D"), z=x.get("z"), delta_bias=x.get("delta_bias"))
    h0 = x.get("h0")
    hl = torch.full_like(h0, float("nan")) if h0 is not None else None
    y, ck = ms.scan_fwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"], **opt,
                                   softplus=softplus, h0=h0, h_last=hl, **kw)
    g = ms.scan_bwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], ck, **opt,
                               softplus=softplus, dh_last=x.get("dh_last"), **kw)
    hl2 = torch.full_like(h0, float("nan")) if h0 is not None else None
    y2 = ms.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], **opt, softplus=softplus,
                     h0=h0, h_last=hl2, **kw)
    g2 = ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], **opt,
                     softplus=softplus, h0=h0, dh_last=x.get("dh_last"), **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "y differs from ms_scan_fwd"
    if h0 is not None:
        assert torch.equal(hl, hl2), "h_last differs from ms_scan_fwd"
    for k in GRADS:
        if g[k] is not None:
            assert torch.equal(g[k], g2[k]), f"{k} differs from ms_scan_bwd"
    return y, ck, g


def _check_states(x, ck, disc, softplus=True):
    """Checkpoint entries against the oracle's state after 16k steps."""
    L = x["u"].shape[1]
    nblk = (L + 15) // 16
    h0 = x.get("h0")
    first = ck[:, 0]
    assert torch.equal(first, h0 if h0 is not None else torch.zeros_like(first))
    for k in sorted({1, nblk // 2, nblk - 1} - {0}):
        t = 16 * k
        pre = {n: (x[n][:, :t].contiguous() if x.get(n) is not None else None)
               for n in ("u", "delta", "B", "C", "z")}
        _, ref_h = oracle.scan(pre["u"], pre["delta"], x["A"], pre["B"], pre["C"],
                               D=x.get("D"), z=pre["z"], delta_bias=x.get("delta_bias"),
                               h0=h0, softplus=softplus, **disc_kw(disc))
        assert_within(ck[:, k], ref_h, "f32", f"checkpoint block {k}")


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("shape", ROWS, ids=lambda s: "B{}L{}D{}N{}{}".format(*s))
def test_checkpoint_pair(gpu, shape, disc):
    batch, L, Dn, N, io = shape
    x = _inputs(batch, L, Dn, N, io, seed=51)
    _, ck, got = _pair(gpu, x, disc)
    _check_states(x, ck, disc)
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], D=x.get("D"),
                          z=x.get("z"), delta_bias=x.get("delta_bias"), h0=x.get("h0"),
                          dh_last=x.get("dh_last"), softplus=True, **disc_kw(disc))
    for k in ("du", "ddelta", "dz"):
        if ref[k] is not None:
            _check(got[k], ref[k], io, k)
    for k in ("dA", "dB", "dC", "dD", "dbias", "dh0"):
        if ref[k] is not None:
            _check(got[k], ref[k], "f32", k)


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "raw_step"])
def test_checkpoint_pair_options_off(gpu, softplus):
    """No gate, D, bias, h0 or dh_last: the first checkpoint is zero."""
    x = _inputs(4, 70, 2048, 16, "bf16", seed=52, optional=False)
    if not softplus:
        x["delta"] = (x["delta"].float().abs() * 0.05 + 0.01).to(x["delta"].dtype)
    _, ck, _ = _pair(gpu, x, "zoh", softplus=softplus)
    _check_states(x, ck, "zoh", softplus=softplus)


@pytest.mark.parametrize("disc", DISCS)
def test_checkpoint_pair_130m_layer(gpu, disc):
    """The 130M-layer workload (B8 L2048 D1536 N16, bf16) in the launch
    configuration the benchmark times: outputs, states and every gradient
    bit-identical to the recomputing pair (which the backward tests hold to
    the oracle at this size); two checkpoint blocks against the oracle on
    sampled channels."""
    w = synth.workload("m130m")
    x = synth.scan_inputs(w, device=DEV, seed=0)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    x["dy"] = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV).to(x["u"].dtype)
    _, ck, _ = _pair(gpu, x, disc)
    ii = torch.arange(0, w.Dn, 97, device=DEV)
    for k in (1, 127):
        t = 16 * k
        _, ref_h = oracle.scan(x["u"][:, :t].index_select(2, ii), x["delta"][:, :t].index_select(2, ii),
                               x["A"].index_select(0, ii), x["B"][:, :t].contiguous(),
                               x["C"][:, :t].contiguous(), D=x["D"].index_select(0, ii),
                               z=x["z"][:, :t].index_select(2, ii),
                               delta_bias=(x["delta_bias"].index_select(0, ii)
                                           if x.get("delta_bias") is not None else None),
                               softplus=w.softplus, **disc_kw(disc))
        assert_within(ck[:, k].index_select(1, ii), ref_h, "f32", f"checkpoint block {k}")
    del x, ck
    torch.cuda.empty_cache()


def test_checkpoint_unsupported_shape(gpu):
    """Few channels: the pair does not serve the shape and says so."""
    x = _inputs(1, 40, 64, 16, "bf16", seed=53)
    assert gpu.checkpoint_bytes(1, 40, 64, 16, gpu.MS_BF16) == 0
    with pytest.raises(gpu.MsError):
        gpu.scan_fwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"])


def test_selective_scan_saved_states(gpu):
    """The autograd function with and without the saved block states gives
    the same output and gradients."""
    x = _inputs(4, 70, 2048, 16, "bf16", seed=54)
    outs = []
    for save in (True, False):
        leaves = {k: x[k].detach().clone().requires_grad_(True)
                  for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
        y = gpu.selective_scan(leaves["u"], leaves["delta"], leaves["A"], leaves["B"],
                               leaves["C"], leaves["D"], leaves["z"], leaves["delta_bias"],
                               leaves["h0"], save_states=save)
        y.backward(x["dy"])
        torch.cuda.synchronize()
        outs.append((y.detach(), {k: v.grad for k, v in leaves.items()}))
    assert torch.equal(outs[0][0], outs[1][0])
    for k, v in outs[0][1].items():
        assert torch.equal(v, outs[1][1][k]), k
