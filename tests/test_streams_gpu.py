"""Calls on different streams run concurrently and independently: the
library keeps no global mutable state besides its thread-local error text,
and every call works on the stream it is given.  Two scans (with their own
workspaces) and a decode step are issued on three streams at once, several
times, and each result must equal the same call run alone, bit for bit."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_three_streams_at_once(gpu):
    w1 = synth.workload("tiny", batch=4, L=1500, Dn=256, N=16, io="bf16")
    w2 = synth.workload("tiny", batch=2, L=700, Dn=192, N=8, io="f32")
    x1 = synth.scan_inputs(w1, device=DEV, seed=101)
    x2 = synth.scan_inputs(w2, device=DEV, seed=102)
    wd = synth.workload("decode", batch=16, Dn=512, steps=1)
    xd = synth.decode_inputs(wd, device=DEV, seed=103)

    def ws(w, x):
        io = gpu.MS_BF16 if x["u"].dtype == torch.bfloat16 else gpu.MS_F32
        n = gpu.workspace_bytes(w.batch, w.L, w.Dn, w.N, io, gpu.flags(True))
        return torch.empty(max(1, n), dtype=torch.uint8, device=DEV)

    ws1, ws2 = ws(w1, x1), ws(w2, x2)

    def scan(x, y, wsp, stream):
        gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                     delta_bias=x.get("delta_bias"), y=y, workspace=wsp, stream=stream)

    def step(h, y, stream):
        gpu.state_update(h, xd["x"][0], xd["delta"][0], xd["A"], xd["B"][0], xd["C"][0],
                         D=xd["D"], z_t=xd["z"][0], delta_bias=xd.get("delta_bias"), y_t=y,
                         stream=stream)

    r1, r2, rd = torch.empty_like(x1["u"]), torch.empty_like(x2["u"]), torch.empty_like(xd["x"][0])
    rh = xd["h0"].clone()
    main = torch.cuda.current_stream()
    scan(x1, r1, ws1, main)
    scan(x2, r2, ws2, main)
    step(rh, rd, main)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        y1, y2, yd = torch.full_like(r1, float("nan")), torch.full_like(r2, float("nan")), \
            torch.full_like(rd, float("nan"))
        h = xd["h0"].clone()
        torch.cuda.synchronize()
        scan(x1, y1, ws1, streams[0])
        scan(x2, y2, ws2, streams[1])
        step(h, yd, streams[2])
        torch.cuda.synchronize()
        assert torch.equal(y1, r1), rep
        assert torch.equal(y2, r2), rep
        assert torch.equal(yd, rd) and torch.equal(h, rh), rep
