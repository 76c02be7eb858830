"""Seeded random shapes across every planner route, against the fp64 oracle.

Each case draws batch, L, d_inner, d_state (weighted toward the boundaries
where the planner changes kernels: 8/9, 16/17, 32/33, 64/65 states, the
row kernels' channel counts), the io type and the discretisation, keeps the
oracle's work under ~4e6 state-steps, and compares y and h_last (from a
random h0) with the tolerances of the other parity tests.  Where the
checkpointed training pair serves the shape, its y and gradients must also
equal the recomputing pair's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, disc_kw

pytestmark = pytest.mark.gpu
DEV = "cuda"
STATES = [1, 3, 4, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32, 33, 40, 48, 63, 64, 65, 80, 100, 127,
          128]
BUDGET = 4_000_000  # batch * L * d_inner * d_state


def _shape(i):
    rng = np.random.RandomState(1000 + i)
    N = int(rng.choice(STATES))
    io = "bf16" if rng.rand() < 0.6 else "f32"
    disc = ["euler", "zoh", "bilinear"][rng.randint(3)]
    if rng.rand() < 0.4:  # enough channels for the row kernels (and the wide rows)
        batch = int(rng.randint(1, 5))
        Dn = int(rng.choice([2048, 2056, 2052, 4096, 4100, 8192, 8200]))
        Dn -= Dn % (8 if io == "bf16" else 4) if rng.rand() < 0.8 else 0
    else:
        batch = int(rng.randint(1, 4))
        Dn = int(rng.randint(1, 300))
    Dn = max(Dn, 1)
    lmax = max(1, BUDGET // (batch * Dn * N))
    L = int(rng.randint(1, min(lmax, 2500) + 1))
    return batch, L, Dn, N, io, disc


# plus shapes the checkpointed pair serves (d_state 9..16, >= 512 tiles)
CASES = [_shape(i) for i in range(40)] + [(4, 20, 2048, 16, "bf16", "zoh"),
                                          (2, 33, 4100, 12, "f32", "euler"),
                                          (1, 40, 8200, 9, "bf16", "bilinear")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}N{}{}-{}".format(*c))
def test_random_shape(gpu, case):
    batch, L, Dn, N, io, disc = case
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, N=N, io=io)
    x = synth.scan_inputs(w, device=DEV, seed=17)
    g = torch.Generator(device=DEV)
    g.manual_seed(18)
    h0 = torch.randn(batch, Dn, N, generator=g, device=DEV)
    h_last = torch.full_like(h0, float("nan"))
    y = gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                     delta_bias=x.get("delta_bias"), h0=h0, h_last=h_last, **disc_kw(disc))
    torch.cuda.synchronize()
    yr, hr = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                         delta_bias=x.get("delta_bias"), h0=h0, **disc_kw(disc))
    assert_within(y, yr, io)
    assert_within(h_last, hr, "f32", "h_last")
    io_code = gpu.MS_BF16 if io == "bf16" else gpu.MS_F32
    if gpu.checkpoint_bytes(batch, L, Dn, N, io_code, gpu.flags(True, **disc_kw(disc))) == 0:
        return
    dy = torch.randn(batch, L, Dn, generator=g, device=DEV).to(x["u"].dtype)
    opt = dict(D=x["D"], z=x["z"], delta_bias=x.get("delta_bias"), **disc_kw(disc))
    y2, ck = gpu.scan_fwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"], h0=h0, **opt)
    ga = gpu.scan_bwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, ck, **opt)
    gb = gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, h0=h0, **opt)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)
    for k, v in ga.items():
        if v is not None:
            assert torch.equal(v, gb[k]), k
