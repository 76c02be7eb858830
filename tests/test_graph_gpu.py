"""The library's calls can be captured in a HIP graph: they allocate nothing,
never synchronise and issue no memset, and every kernel argument is fixed at
launch.  Each test captures a call with preallocated outputs and workspace,
replays the graph several times with eager work and synchronisations between
the replays, and checks every replay bit for bit against the same call run
eagerly (the library is deterministic)."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _scan_inputs(seed):
    w = synth.workload("tiny", batch=2, L=1000, Dn=192, N=16, io="bf16")
    return w, synth.scan_inputs(w, device=DEV, seed=seed)


def test_scan_fwd_in_a_graph(gpu):
    w, x = _scan_inputs(71)
    io = gpu.MS_BF16
    ws = torch.empty(max(1, gpu.workspace_bytes(w.batch, w.L, w.Dn, w.N, io, gpu.flags(True))),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty_like(x["u"])
    h_last = torch.empty(w.batch, w.Dn, w.N, device=DEV)

    def call(out, hl):
        gpu.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                     delta_bias=x.get("delta_bias"), y=out, h_last=hl, workspace=ws)

    ref_y, ref_h = torch.empty_like(y), torch.empty_like(h_last)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(ref_y, ref_h)  # eager, also the warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y, h_last)
    for i in range(4):
        y.fill_(float("nan"))
        h_last.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y), f"replay {i}"
        assert torch.equal(h_last, ref_h), f"replay {i}"
        call(ref_y, ref_h)  # eager work between replays (same result)
        torch.cuda.synchronize()


def test_decode_steps_in_a_graph(gpu):
    """Eight decode steps captured as one graph, replayed from the same state."""
    w = synth.workload("decode", batch=32, Dn=256, steps=8)
    x = synth.decode_inputs(w, device=DEV, seed=72)
    h0 = x["h0"].clone()
    ys = [torch.empty_like(x["x"][0]) for _ in range(w.steps)]

    def steps(h, outs):
        for t in range(w.steps):
            gpu.state_update(h, x["x"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t],
                             D=x["D"], z_t=x["z"][t], delta_bias=x.get("delta_bias"),
                             y_t=outs[t])

    h_ref = h0.clone()
    ys_ref = [torch.empty_like(y) for y in ys]
    steps(h_ref, ys_ref)
    torch.cuda.synchronize()
    h = h0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(h, ys)
    for i in range(3):
        h.copy_(h0)
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), f"replay {i}"
        for t in range(w.steps):
            assert torch.equal(ys[t], ys_ref[t]), f"replay {i} step {t}"


def test_scan_bwd_in_a_graph(gpu):
    w, x = _scan_inputs(73)
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(74)
    dy = torch.randn(w.batch, w.L, w.Dn, generator=g0, device=DEV).to(x["u"].dtype)
    io = gpu.MS_BF16
    ws = torch.empty(gpu.scan_bwd_workspace_bytes(w.batch, w.L, w.Dn, w.N, io, gpu.flags(True)),
                     dtype=torch.uint8, device=DEV)

    def call():
        return gpu.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                            delta_bias=x.get("delta_bias"), workspace=ws)

    ref = call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items() if v is not None}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    for i in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), f"replay {i}: {k}"
        call()  # eager work between replays
        torch.cuda.synchronize()
