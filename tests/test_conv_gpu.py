"""GPU parity of ms_conv1d_silu (causal depthwise conv1d + silu, the step that
produces the scan input) against the fp64 oracle, through the C ABI, on the
same seeded inputs; and conv -> scan end to end."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(ms, x, silu=True):
    u = ms.conv1d_silu(x["x"], x["weight"], x.get("bias"), x.get("x_prev"), silu=silu)
    torch.cuda.synchronize()
    return u


def _ref(x, silu=True):
    return oracle.conv1d(x["x"], x["weight"], x.get("bias"), x.get("x_prev"), silu=silu)


SHAPES = [
    # batch, L, Dn, width, io
    (1, 1, 4, 4, "f32"),
    (2, 37, 8, 4, "bf16"),
    (3, 100, 70, 3, "f32"),     # d_inner not a multiple of 4: one channel per lane
    (1, 33, 65, 1, "bf16"),
    (2, 257, 256, 4, "bf16"),   # several time chunks and a ragged last chunk
    (1, 70, 12, 8, "f32"),
    (2, 64, 1536, 2, "bf16"),
    (1, 300, 260, 5, "bf16"),
]


@pytest.mark.parametrize("history", [False, True], ids=["zeros", "x_prev"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}L{}D{}W{}{}".format(*s))
def test_conv_edge_shapes(gpu, shape, history):
    batch, L, Dn, width, io = shape
    w = synth.workload("tiny", batch=batch, L=L, Dn=Dn, io=io)
    x = synth.conv_inputs(w, width, device=DEV, seed=2, history=history)
    for silu in (True, False):
        assert_within(_run(gpu, x, silu), _ref(x, silu), io, f"silu={silu}")


def test_conv_without_bias(gpu):
    w = synth.workload("tiny", batch=2, L=50, Dn=36, io="bf16")
    x = synth.conv_inputs(w, 4, device=DEV, seed=3)
    del x["bias"]
    assert_within(_run(gpu, x), _ref(x), "bf16")


def test_conv_pieces_equal_whole(gpu):
    """Two pieces, the second given the last width-1 inputs of the first as
    x_prev, give bit-identical results to one call over the whole sequence."""
    w = synth.workload("m130m", batch=2, L=300, Dn=192)
    x = synth.conv_inputs(w, 4, device=DEV, seed=4)
    whole = _run(gpu, x)
    L1 = 113
    p1 = {"x": x["x"][:, :L1].contiguous(), "weight": x["weight"], "bias": x["bias"]}
    p2 = {"x": x["x"][:, L1:].contiguous(), "weight": x["weight"], "bias": x["bias"],
          "x_prev": x["x"][:, L1 - 3:L1].contiguous()}
    got = torch.cat([_run(gpu, p1), _run(gpu, p2)], dim=1)
    assert torch.equal(got, whole)


def test_conv_130m_layer_full(gpu):
    w = synth.workload("m130m")
    x = synth.conv_inputs(w, 4, device=DEV, seed=0)
    u = _run(gpu, x)
    assert_within(u, _ref(x), "bf16")


def test_conv_then_scan_end_to_end(gpu):
    """u = conv1d_silu(x) on the GPU, then the scan of u: u against the oracle's
    conv, and y against the oracle's scan of that same bf16 u (the io type the
    GPU hands from one call to the next)."""
    w = synth.workload("m130m", batch=2, L=512, Dn=256)
    s = synth.scan_inputs(w, device=DEV, seed=5)
    c = synth.conv_inputs(w, 4, device=DEV, seed=5)
    u = _run(gpu, c)
    y = gpu.scan_fwd(u, s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                     delta_bias=s.get("delta_bias"))
    torch.cuda.synchronize()
    assert_within(u, _ref(c), "bf16", "u")
    yr, _ = oracle.scan(u.cpu(), s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                        delta_bias=s.get("delta_bias"))
    assert_within(y, yr, "bf16")
