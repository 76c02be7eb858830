"""selective_scan as a torch autograd operation: its forward equals
scan_fwd bit for bit, and the gradients torch's backward delivers (through
ms_scan_bwd) match the fp64 oracle's backward for the same output gradient,
to the backward's bound: |g - ref| <= 2e-4 (|ref| + rms(ref))."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import DISCS, disc_kw

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _close(got, ref, what, rtol=2e-4):
    got = got.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    lim = rtol * (np.abs(ref) + rms) + 1e-30
    bad = ~(np.abs(got - ref) <= lim)
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} outside bound"


@pytest.mark.parametrize("disc", DISCS)
def test_autograd_gradients_match_oracle(gpu, disc):
    w = synth.workload("tiny", batch=2, L=150, Dn=70, N=16, io="f32")
    x = synth.scan_inputs(w, device=DEV, seed=81)
    g = torch.Generator(device=DEV)
    g.manual_seed(82)
    x["delta_bias"] = torch.randn(w.Dn, generator=g, device=DEV) * 0.3
    x["h0"] = torch.randn(w.batch, w.Dn, w.N, generator=g, device=DEV)
    wy = torch.randn(w.batch, w.L, w.Dn, generator=g, device=DEV)
    names = ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0"]
    leaf = {k: x[k].clone().requires_grad_(True) for k in names}
    kw = disc_kw(disc)
    y = gpu.selective_scan(leaf["u"], leaf["delta"], leaf["A"], leaf["B"], leaf["C"],
                           D=leaf["D"], z=leaf["z"], delta_bias=leaf["delta_bias"],
                           h0=leaf["h0"], **kw)
    y_plain = gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                           delta_bias=x["delta_bias"], h0=x["h0"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y_plain)
    (y * wy).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], wy, D=x["D"], z=x["z"],
                          delta_bias=x["delta_bias"], h0=x["h0"], softplus=True, **kw)
    pairs = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "z": "dz", "delta_bias": "dbias", "h0": "dh0"}
    for k, gk in pairs.items():
        assert leaf[k].grad is not None, k
        _close(leaf[k].grad, ref[gk], f"{k} ({disc})")


def test_autograd_bf16_and_optional_terms(gpu):
    """bf16 io without D, z, bias or h0: the io gradients come back in bf16."""
    w = synth.workload("tiny", batch=1, L=300, Dn=64, N=16, io="bf16")
    x = synth.scan_inputs(w, device=DEV, seed=83)
    u = x["u"].clone().requires_grad_(True)
    B = x["B"].clone().requires_grad_(True)
    A = x["A"].clone().requires_grad_(True)
    y = gpu.selective_scan(u, x["delta"], A, B, x["C"])
    y.float().sum().backward()
    torch.cuda.synchronize()
    assert u.grad.dtype == torch.bfloat16 and B.grad.dtype == torch.bfloat16
    assert A.grad.dtype == torch.float32
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"],
                          np.ones((w.batch, w.L, w.Dn)), softplus=True)
    _close(A.grad, ref["dA"], "dA")
    # bf16-rounded gradients: the rounding bound (2^-8 relative) on top
    gu = u.grad.double().cpu().numpy()
    assert np.all(np.abs(gu - ref["du"]) <= 2.0 ** -8 * np.abs(ref["du"]) + 2e-4 *
                  (np.abs(ref["du"]) + np.sqrt(np.mean(ref["du"] ** 2))))
