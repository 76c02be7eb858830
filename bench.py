#!/usr/bin/env python3
"""Benchmark of the selective scan (S6) hot path on one MI355X.

One step = one ms_scan_fwd call over one batch of the Mamba-130M-layer
workload (batch 8, L 2048, d_inner 1536, d_state 16, bf16 io, fp32 state,
Euler, softplus + bias, z gate and D skip on), inputs resident in HBM.
Several input/output buffer sets are rotated so that consecutive steps do
not find the previous step's data in the 256 MB Infinity Cache.

Prints ONE JSON line: elements/s (B*L*d_inner per second); the dominant
kernel's roofline position, from its HIP-event kernel times recorded on the
launch stream over the timed region (ms_profile_*); the whole call's HBM
rate against the 8 TB/s peak and its VALU fraction; line items for the 3B
layer (Euler, ZOH, bilinear), the long-context d_state 64 scan (with its
exponential rate against the measured v_exp_f32 rate), the wide-state scans
(d_state 128 Euler, d_state 64 ZOH; batch 2, L 8192, d_inner 1536), decode, conv1d,
backward and the fused step projection; the chip rates measured by
libmsprobe (v_exp_f32, fp32 FMA, copy and read bandwidth); and the fp64 CPU
oracle timed on this host's cores on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Warm-up: at least --warmup untimed calls and at least --warm-seconds of
them, so the GPU clock has ramped before the timed calls (kernel times fall
by ~10% over the first ~20 ms of load).

Profile helpers (used to write the summaries kept under profiles/):
    python bench.py --steps 3 --warmup 1 --no-cpu --no-secondary --copy-calibration
        (the command run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)
    python bench.py --rocprof-summary KTRACE_DIR [--fetch DIR --write DIR]
        (no GPU: reads rocprofv3 CSV output and prints a markdown summary)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan elem/s (B·L·D_inner) + achieved HBM GB/s vs peak, 130M & 3B layer shapes"
HBM_PEAK_GBPS = 8000.0
# Peak VALU rate of the chip for fp32 lane-operations (an FMA counted as one
# operation): the published 157.3 TFLOP/s fp32 vector figure is 2 flops x
# 78.6e12 FMA/s = 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz.  Plain VOP2
# instructions reach it without packed math: libmsprobe measures ~1.5 wave64
# FMAs per SIMD per 4 cycles, i.e. two 16-lane passes overlap; DPP and
# transcendental instructions do not (rates in the bench line's "rates").
VALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
COPY_MIB = 256  # size of the calibration copy (read and written)
# the pass that writes y: scan_row with SUMMARY (its 4th argument) false,
# scan_lane with SUMMARY (its 7th) false, or scan_tile with SUMMARY (its last) false
MAIN_KERNEL_RE = (r"scan_row<(?:[^,>]*, ){3}false[,>]|scan_lane<(?:[^,>]*, ){6}false[,>]|"
                  r"scan_tile<[^>]*false>")
WORKLOAD_TITLE = {"m130m": "Mamba-130M-layer selective scan (S6) forward",
                  "m3b": "Mamba-3B-layer selective scan (S6) forward",
                  "long": "long-context selective scan (S6) forward, d_state 64",
                  "wide128": "wide-state selective scan (S6) forward, d_state 128",
                  "wide64": "wide-state selective scan (S6) forward, d_state 64"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=0.25,
                    help="minimum wall time of the untimed warm-up calls")
    ap.add_argument("--workload", default="m130m", choices=["m130m", "m3b", "long", "wide128", "wide64"])
    ap.add_argument("--zoh", action="store_true", help="zero-order hold instead of Euler")
    ap.add_argument("--bilinear", action="store_true", help="bilinear instead of Euler")
    ap.add_argument("--buffer-sets", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle sample")
    ap.add_argument("--no-secondary", action="store_true", help="skip the line items")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run a {COPY_MIB} MiB device copy (HBM counter calibration)")
    ap.add_argument("--rocprof-summary", metavar="KTRACE_DIR",
                    help="summarise rocprofv3 output instead of benchmarking")
    ap.add_argument("--fetch", metavar="DIR", help="rocprofv3 --pmc FETCH_SIZE output dir")
    ap.add_argument("--write", metavar="DIR", help="rocprofv3 --pmc WRITE_SIZE output dir")
    ap.add_argument("--counters", metavar="DIR", action="append", default=[],
                    help="other rocprofv3 --pmc output dirs: mean of every counter per kernel")
    return ap.parse_args()


def source_hash() -> str:
    """Hash of everything that decides the kernels' code: sources, header,
    build flags."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "selective_state_space_81_amd", "csrc", "*")))
    files += [os.path.join(ROOT, "include", "msscan.h"),
              os.path.join(ROOT, "selective_state_space_81_amd", "build.py")]
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- counting --
def valu_ops_per_element(n_state: int, disc: str, softplus: bool = True) -> int:
    """fp32 VALU operations the method needs per element (b, t, d), counted
    one per lane-instruction, an FMA as one:
      per state: dt*A, exp, B*x (Euler x = dt*u), A_bar*h + .., C*h + ..  = 5
                 ZOH adds (A_bar - 1)/A as one FMA with 1/A kept, and one
                 more product with B*u                                   = 7
                 bilinear: dt*A, 1 - ../2, reciprocal r, A_bar = 2r - 1,
                 x*r, B*.., A_bar*h + .., C*h + ..                        = 8
      per element: delta + bias, softplus (exp, 1 +, log), dt*u (Euler),
                 D*u + y, silu gate (exp, 1 +, reciprocal, z*r), y*gate.
    Only the kernel that writes y is priced this way; the segment-summary
    pass is work the parallel split adds, not work of the method."""
    per_state = {"euler": 5, "zoh": 7, "bilinear": 8}[disc]
    per_elem = 1 + (3 if softplus else 0) + (0 if disc == "zoh" else 1) + 1 + 4 + 1
    return per_state * n_state + per_elem


def bwd_ops_per_element(n_state: int) -> int:
    """Minimum fp32 VALU operations of the backward's per-segment pass (Euler,
    softplus, gate, D), counted as in valu_ops_per_element: one forward
    recompute (5 per state), the adjoint (l, dB and dC terms, du, the A_bar
    and dt terms of d(dt) and dA, mu: 14 per state), the sums over channels of
    dB and dC (2 per state), and ~30 per element (softplus and its
    derivative, the gate and its derivative, D, the stores' conversions)."""
    return 21 * n_state + 30


# ----------------------------------------------------------------- timing --
def make_sets(w, n_sets):
    import torch
    import synth
    base = synth.scan_inputs(w, device="cuda", seed=0)
    sets = []
    for i in range(n_sets):
        x = base if i == 0 else {k: v.clone() for k, v in base.items()}
        sets.append((x, torch.empty_like(base["u"])))
    return sets


def warm_up(call, n, seconds):
    """At least n untimed calls, and at least `seconds` of them."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < seconds:
        call(i)
        i += 1
        if i % 16 == 0 or i >= n:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_calls(ms, sets, w, steps, warmup, zoh=False, bilinear=False, warm_seconds=0.25):
    """Two timed regions of `steps` ms_scan_fwd calls each, on the stream the
    calls are enqueued on (torch's current stream):
      1. plain calls, bracketed by torch events -> ms per call (the value);
      2. the same calls with the library's kernel timing on (ms_profile_*):
         HIP events recorded on that stream around each kernel launch give the
         per-phase kernel times.  The event records add gaps between kernels,
         so region 2 is not used for the per-call time."""
    import torch
    stream = torch.cuda.current_stream()
    io = ms.MS_BF16 if w.io == "bf16" else ms.MS_F32
    ws_n = ms.workspace_bytes(w.batch, w.L, w.Dn, w.N, io, ms.flags(w.softplus, zoh, bilinear))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def call(i):
        x, y = sets[i % len(sets)]
        ms.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                    delta_bias=x.get("delta_bias"), softplus=w.softplus, zoh=zoh,
                    bilinear=bilinear, y=y, workspace=ws if ws_n else None, stream=stream)

    warm_up(call, warmup, warm_seconds)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    t_ms = start.elapsed_time(end) / steps
    ms.profile_begin(steps)
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    phases = ms.profile_end()
    return t_ms, phases


def copy_calibration(reps=3):
    """A plain device copy of COPY_MIB MiB (one read and one write of every
    byte), so that a counter run can scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = COPY_MIB * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def decode_bytes(w) -> int:
    """Bytes one ms_state_update step must move: h read and written
    ([batch, Dn, N] fp32), x, delta, z read and y written ([batch, Dn] io),
    B_t and C_t read ([batch, N] io), A ([Dn, N]) and D, delta_bias ([Dn])."""
    e = 2 if w.io == "bf16" else 4
    return (2 * w.batch * w.Dn * w.N * 4 + 4 * w.batch * w.Dn * e + 2 * w.batch * w.N * e
            + w.Dn * w.N * 4 + 2 * w.Dn * 4)


def measure_decode(ms, reps=3):
    """The decode workload: w.steps back-to-back ms_state_update calls on a
    state resident in HBM; ms per step over `reps` timed runs, plus the
    step kernel's HIP-event time."""
    import torch
    import synth
    w = synth.workload("decode")
    x = synth.decode_inputs(w, device="cuda", seed=0)
    h = x["h0"].clone()
    y = torch.empty_like(x["x"][0])
    stream = torch.cuda.current_stream()

    def run():
        for t in range(w.steps):
            ms.state_update(h, x["x"][t], x["delta"][t], x["A"], x["B"][t], x["C"][t], D=x["D"],
                            z_t=x["z"][t], delta_bias=x.get("delta_bias"), softplus=w.softplus,
                            y_t=y, stream=stream)

    run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    t_ms = start.elapsed_time(end) / (reps * w.steps)
    ms.profile_begin(w.steps)
    run()
    torch.cuda.synchronize()
    k_ms = ms.profile_end()["step"]["mean_ms"]
    nb = decode_bytes(w)
    return {"workload": f"recurrent decode, ms_state_update: batch {w.batch}, d_inner {w.Dn}, "
                        f"d_state {w.N}, {w.io} io, fp32 state in HBM, {w.steps} steps",
            "ms_per_step": t_ms, "kernel_ms": k_ms, "bytes_per_step": nb,
            "hbm_gbps": nb / (t_ms * 1e-3) / 1e9,
            "hbm_frac": nb / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "kernel_hbm_gbps": nb / (k_ms * 1e-3) / 1e9}


def measure_conv(ms, reps=20, width=4):
    """ms_conv1d_silu on the 130M-layer shape (B8 L2048 D1536, bf16, width
    4, bias, silu): ms per call over rotated buffers, kernel time from HIP
    events, and the HBM rate of its algorithmic bytes (x read, u written,
    weight and bias read)."""
    import torch
    import synth
    w = synth.workload("m130m")
    sets = []
    for i in range(4):
        c = synth.conv_inputs(w, width, device="cuda", seed=i)
        sets.append((c, torch.empty_like(c["x"])))
    stream = torch.cuda.current_stream()

    def call(i):
        c, u = sets[i % len(sets)]
        ms.conv1d_silu(c["x"], c["weight"], c["bias"], None, u=u, stream=stream)

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(reps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    t_ms = start.elapsed_time(end) / reps
    ms.profile_begin(reps)
    for i in range(reps):
        call(i)
    torch.cuda.synchronize()
    k_ms = ms.profile_end()["conv"]["mean_ms"]
    e = 2 if w.io == "bf16" else 4
    nb = 2 * w.batch * w.L * w.Dn * e + w.Dn * (width + 1) * 4
    del sets
    # the same bytes moved by a plain copy (libmsprobe's 16-byte copy, x-sized
    # source to u-sized destination, rotated over 4 pairs like the conv):
    # the rate an op of this size can reach on this machine
    c_ms = copy_ms(w.batch * w.L * w.Dn * e, reps)
    c_gbps = 2 * w.batch * w.L * w.Dn * e / (c_ms * 1e-3) / 1e9
    gbps = nb / (t_ms * 1e-3) / 1e9
    return {"workload": f"causal depthwise conv1d + silu (ms_conv1d_silu): batch {w.batch}, "
                        f"L {w.L}, d_inner {w.Dn}, width {width}, {w.io}",
            "ms_per_call": t_ms, "kernel_ms": k_ms, "bytes_per_call": nb,
            "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
            "kernel_hbm_gbps": nb / (k_ms * 1e-3) / 1e9,
            "same_size_copy_ms": c_ms, "same_size_copy_gbps": c_gbps,
            "frac_of_same_size_copy": gbps / c_gbps}


def copy_ms(nbytes, reps):
    """ms per call of libmsprobe's copy of nbytes (a multiple of 16) into
    another buffer, over 4 rotated source/destination pairs, timed back to
    back like the ops it is set beside."""
    import ctypes
    import torch
    from selective_state_space_81_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.msprobe_copy.argtypes = [vp, vp, i64, i32, vp]
    words = nbytes // 16
    pairs = [(torch.ones(nbytes // 4, dtype=torch.float32, device="cuda"),
              torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")) for _ in range(4)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    blocks = max(1, min(16384, (words + 255) // 256))

    def call(i):
        s, d = pairs[i % len(pairs)]
        rc = lib.msprobe_copy(s.data_ptr(), d.data_ptr(), words, blocks, sp)
        if rc != 0:
            raise RuntimeError(f"probe copy failed: {rc}")

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(reps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / reps
    del pairs
    return t


def measure_bwd(ms, reps=20, warm=3):
    """ms_scan_bwd (gradients of every input) on the 130M-layer workload:
    ms per call (forward recompute included) and the main backward kernel's
    HIP-event time."""
    import torch
    import synth
    w = synth.workload("m130m")
    x = synth.scan_inputs(w, device="cuda", seed=0)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dy = torch.randn(w.batch, w.L, w.Dn, generator=g, device="cuda").to(x["u"].dtype)
    io = ms.MS_BF16 if w.io == "bf16" else ms.MS_F32
    ws = torch.empty(ms.scan_bwd_workspace_bytes(w.batch, w.L, w.Dn, w.N, io,
                                                 ms.flags(w.softplus)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                    delta_bias=x.get("delta_bias"), softplus=w.softplus, workspace=ws,
                    stream=stream)

    warm_up(lambda i: call(), warm, 0.25)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    t_ms = start.elapsed_time(end) / reps
    ms.profile_begin(reps)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    ph = ms.profile_end()
    elems = w.batch * w.L * w.Dn
    main_ms = ph["main"]["mean_ms"]

    def other(zoh, bilinear):  # the same call with the other discretisations
        ws2 = torch.empty(ms.scan_bwd_workspace_bytes(
            w.batch, w.L, w.Dn, w.N, io, ms.flags(w.softplus, zoh, bilinear)),
            dtype=torch.uint8, device="cuda")

        def c():
            ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                        delta_bias=x.get("delta_bias"), softplus=w.softplus, zoh=zoh,
                        bilinear=bilinear, workspace=ws2, stream=stream)

        warm_up(lambda i: c(), warm, 0.25)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(reps):
            c()
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    t_zoh, t_bil = other(True, False), other(False, True)
    wide = measure_bwd_wide(ms)
    ckpt = measure_checkpointed_pair(ms, w, x, dy, reps, warm)
    return {"wide_state": wide, "checkpointed": ckpt,
            "workload": "gradients of the Mamba-130M-layer scan (ms_scan_bwd: du, ddelta, dz, "
                        "dA, dB, dC, dD, dbias, dh0), Euler, bf16",
            "zoh_ms_per_call": t_zoh, "bilinear_ms_per_call": t_bil,
            "ms_per_call": t_ms, "elem_per_s": elems / (t_ms * 1e-3),
            "main_ops_per_element": bwd_ops_per_element(w.N),
            "main_valu_frac": bwd_ops_per_element(w.N) * elems / (main_ms * 1e-3) / 1e12
                              / VALU_PEAK_TOPS,
            "kernels_ms": {k: v["per_call_ms"] for k, v in ph.items()
                           if k != "calls" and v["launches"]}}


def measure_checkpointed_pair(ms, w, x, dy, reps, warm):
    """The training pair with forward-saved checkpoints
    (ms_scan_fwd_checkpoint + ms_scan_bwd_checkpoint) on workload w, beside
    the recomputing pair (ms_scan_fwd + ms_scan_bwd): ms per call of each,
    in the three discretisations, and the checkpointed backward's kernel
    times."""
    import torch
    io = ms.MS_BF16 if w.io == "bf16" else ms.MS_F32
    stream = torch.cuda.current_stream()
    y = torch.empty_like(x["u"])
    ck = torch.empty(w.batch, (w.L + 15) // 16, w.Dn, w.N, dtype=torch.float32, device="cuda")
    opt = dict(D=x["D"], z=x["z"], delta_bias=x.get("delta_bias"), softplus=w.softplus)

    def timed(fn):
        warm_up(lambda i: fn(), warm, 0.25)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(reps):
            fn()
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    out = {"checkpoint_bytes": ms.checkpoint_bytes(w.batch, w.L, w.Dn, w.N, io,
                                                   ms.flags(w.softplus))}
    for disc in ("euler", "zoh", "bilinear"):
        kw = dict(zoh=disc == "zoh", bilinear=disc == "bilinear")
        fl = ms.flags(w.softplus, **kw)
        ws = torch.empty(ms.scan_bwd_workspace_bytes(w.batch, w.L, w.Dn, w.N, io, fl),
                         dtype=torch.uint8, device="cuda")
        wsc = torch.empty(ms.scan_bwd_checkpoint_workspace_bytes(w.batch, w.L, w.Dn, w.N, io,
                                                                 fl),
                          dtype=torch.uint8, device="cuda")
        fwd = lambda: ms.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], **opt,  # noqa
                                  **kw, y=y, stream=stream)
        fwd_ck = lambda: ms.scan_fwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"],  # noqa
                                                **opt, **kw, y=y, checkpoint=ck, stream=stream)
        bwd = lambda: ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, **opt,  # noqa
                                  **kw, workspace=ws, stream=stream)
        bwd_ck = lambda: ms.scan_bwd_checkpoint(x["u"], x["delta"], x["A"], x["B"], x["C"],  # noqa
                                                dy, ck, **opt, **kw, workspace=wsc,
                                                stream=stream)
        t = {"fwd_ms": timed(fwd), "fwd_checkpoint_ms": timed(fwd_ck), "bwd_ms": timed(bwd)}
        fwd_ck()
        t["bwd_checkpoint_ms"] = timed(bwd_ck)
        t["pair_recompute_ms"] = t["fwd_ms"] + t["bwd_ms"]
        t["pair_checkpoint_ms"] = t["fwd_checkpoint_ms"] + t["bwd_checkpoint_ms"]
        if disc == "euler":
            ms.profile_begin(reps)
            for _ in range(reps):
                bwd_ck()
            torch.cuda.synchronize()
            ph = ms.profile_end()
            t["bwd_checkpoint_kernels_ms"] = {k: v["per_call_ms"] for k, v in ph.items()
                                              if k != "calls" and v["launches"]}
        out[disc] = t
        del ws, wsc
    return out


def measure_bwd_wide(ms, reps=3):
    """ms_scan_bwd above 16 states: the long-context layer shape shortened to
    L 65536 (B1 D1536 N64, bf16, Euler, no softplus or bias), every
    gradient; ms per call and the phases' kernel times per call."""
    import torch
    import synth
    w = synth.workload("long", L=65536)
    x = synth.scan_inputs(w, device="cuda", seed=0)
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    dy = torch.randn(w.batch, w.L, w.Dn, generator=g, device="cuda").to(x["u"].dtype)
    ws = torch.empty(ms.scan_bwd_workspace_bytes(w.batch, w.L, w.Dn, w.N, ms.MS_BF16,
                                                 ms.flags(w.softplus)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                    delta_bias=x.get("delta_bias"), softplus=w.softplus, workspace=ws,
                    stream=stream)

    call()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(reps):
        call()
    s1.record(stream)
    torch.cuda.synchronize()
    t_ms = s0.elapsed_time(s1) / reps
    ms.profile_begin(reps)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    ph = ms.profile_end()
    elems = w.batch * w.L * w.Dn
    out = {"workload": f"gradients of the long-context scan shape at L {w.L} (B{w.batch} "
                       f"D{w.Dn} N{w.N}, bf16, Euler): d_state 64 in four 16-state slices",
           "ms_per_call": t_ms, "elem_per_s": elems / (t_ms * 1e-3),
           "workspace_bytes": int(ws.numel()),
           "kernels_ms": {k: v["per_call_ms"] for k, v in ph.items()
                          if k != "calls" and v["launches"]}}
    del x, dy, ws
    torch.cuda.empty_cache()
    return out


def measure_dtproj(ms, name="m130m", rank=16, reps=20):
    """ms_scan_fwd_dtproj (Euler) on workload `name` with a rank-`rank` step
    projection (dt_low [batch, L, rank] and W_dt [d_inner, rank], in the io
    dtype): ms per call over rotated buffers and the kernels' HIP-event times.
    Beside it, the same result computed in two steps -- torch's matmul writing
    the raw step in the io dtype, then ms_scan_fwd -- for comparison."""
    import torch
    import synth
    w = synth.workload(name)
    base = synth.scan_inputs(w, device="cuda", seed=0)
    sets = []
    for i in range(4):
        x = dict(base)
        x.update(synth.dtproj_inputs(w, rank, device="cuda", seed=i))
        sets.append((x, torch.empty_like(base["u"])))
    io = ms.MS_BF16 if w.io == "bf16" else ms.MS_F32
    ws = torch.empty(max(1, ms.dtproj_workspace_bytes(w.batch, w.L, w.Dn, w.N, io,
                                               ms.flags(w.softplus))),
                     dtype=torch.uint8, device="cuda")
    # the plain scan's own plan (it may differ from the fused call's)
    ws2 = torch.empty(max(1, ms.workspace_bytes(w.batch, w.L, w.Dn, w.N, io, ms.flags(w.softplus))),
                      dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def fused(i):
        x, y = sets[i % len(sets)]
        ms.scan_fwd_dtproj(x["u"], x["dt_low"], x["W_dt"], x["A"], x["B"], x["C"], D=x["D"],
                           z=x["z"], delta_bias=x.get("delta_bias"), softplus=w.softplus, y=y,
                           workspace=ws, stream=stream)

    delta = torch.empty_like(base["u"])

    def two_step(i):
        x, y = sets[i % len(sets)]
        torch.matmul(x["dt_low"], x["W_dt"].t(), out=delta)
        ms.scan_fwd(x["u"], delta, x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                    delta_bias=x.get("delta_bias"), softplus=w.softplus, y=y, workspace=ws2,
                    stream=stream)

    def timed(fn):
        warm_up(fn, 3, 0.25)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(reps):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    t_fused = timed(fused)
    t_two = timed(two_step)
    ms.profile_begin(reps)
    for i in range(reps):
        fused(i)
    torch.cuda.synchronize()
    ph = ms.profile_end()
    elems = w.batch * w.L * w.Dn
    main_ms = ph["main"]["mean_ms"]
    ops = valu_ops_per_element(w.N, "euler", softplus=w.softplus) * elems
    return {"workload": f"{WORKLOAD_TITLE[name]} with the rank-{rank} step projection "
                        f"fused (ms_scan_fwd_dtproj), Euler, {w.io}",
            "ms_per_call": t_fused, "elem_per_s": elems / (t_fused * 1e-3),
            "two_step_ms_per_call": t_two,
            "two_step": f"torch.matmul (raw step written in {w.io}) + ms_scan_fwd",
            "main_valu_frac": ops / (main_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS,
            "projection_flops_per_call": 2 * rank * elems,
            "kernels_ms": {k: v["per_call_ms"] for k, v in ph.items()
                           if k != "calls" and v["launches"]}}


# ------------------------------------------------------------ CPU oracle --
def cpu_baseline(w, min_seconds, disc="euler"):
    """fp64 oracle on this host's cores on the same workload, compute time
    only: batch rows (full sequence; all channels, or the first `chans` when a
    row is very large) are scanned one after another, cycling over the batch,
    until at least min_seconds have passed."""
    import numpy as np
    import oracle
    import synth
    x = synth.scan_inputs(w, device="cpu", seed=0)
    threads = oracle.max_threads()
    chans = w.Dn if w.L * w.Dn <= (1 << 25) else max(64, (1 << 25) // w.L)
    shared = {k: np.ascontiguousarray(x[k][:chans].double().numpy())
              for k in ("A", "D", "delta_bias") if x.get(k) is not None}
    rows, elapsed, b = 0, 0.0, 0
    while elapsed < min_seconds and rows < 64 * w.batch:
        f = {k: np.ascontiguousarray(x[k][b:b + 1, :, :chans].double().numpy())
             for k in ("u", "delta", "z")}
        f.update({k: np.ascontiguousarray(x[k][b:b + 1].double().numpy()) for k in ("B", "C")})
        t0 = time.perf_counter()
        oracle.scan(f["u"], f["delta"], shared["A"], f["B"], f["C"], D=shared.get("D"), z=f["z"],
                    delta_bias=shared.get("delta_bias"), softplus=w.softplus,
                    zoh=disc == "zoh", bilinear=disc == "bilinear",
                    nthreads=threads)
        elapsed += time.perf_counter() - t0
        rows += 1
        b = (b + 1) % w.batch
    elems = rows * w.L * chans
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    what = f"all {w.Dn} channels" if chans == w.Dn else f"the first {chans} of {w.Dn} channels"
    return {"value": elems / elapsed, "unit": "elem/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} batch rows of the {w.name} workload (each: {what} "
                      f"x L={w.L}, d_state {w.N}, {disc}, "
                      f"softplus {'on' if w.softplus else 'off'}, z gate, D), cycling over "
                      f"its {w.batch} rows; fp64 C oracle, OpenMP over channels, "
                      f"{threads} threads; {elapsed:.1f} s compute; host CPU: {cpu}"}


# --------------------------------------------------------- traffic record --
def load_traffic(w_name: str, src: str):
    """HBM bytes per launch of the dominant kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summary in profiles/, if it was taken on the
    current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"hbm_traffic_scan_main_{w_name}.md")
    if not os.path.exists(p):
        return None
    fields = {}
    with open(p) as fh:
        for line in fh:
            m = re.match(r"^- (\w+): `?([^`\s]+)`?", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_hash") != src:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------- rocprof tools --
def _csv(dirname, suffix):
    hits = sorted(glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirname}")
    with open(hits[0]) as fh:
        return list(csv.DictReader(fh))


def _short(name):
    m = re.search(r"(scan_row<[^>]*>|scan_lane<[^>]*>|scan_tile<[^>]*>|"
                  r"bc_prepare<[^>]*>|carry_chain<[^>]*>|carry_parts<[^>]*>?|step_quads<[^>]*>|"
                  r"conv1d_kernel<[^>]*>|"
                  r"bwd_main<[^>]*>|bwd_row<[^>]*>|seg_summaries<[^>]*>|reduce_bc4_params|reduce_bc4|reduce_bc|"
                  r"wide_\w+(?:<[^>]*>)?|"
                  r"reduce_param_groups|reduce_params|"
                  r"neg_kernel)", name)
    if not m:
        return name[:60]
    k = m.group(1)
    # a name cut at 60 characters before it reached the profiler's csv can
    # lack the template's closing bracket
    return k + ">" if k.startswith("carry_parts<") and not k.endswith(">") else k


def _pmc_per_dispatch(dirname, counter):
    """Mean counter value (KiB) per dispatch, by short kernel name."""
    acc = {}
    for r in _csv(dirname, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        k = _short(r["Kernel_Name"])
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def rocprof_summary(args):
    rows = _csv(args.rocprof_summary, "kernel_stats.csv")
    print("| kernel | calls | average us | min us | max us |")
    print("|---|---|---|---|---|")
    for r in rows:
        n = r["Name"]
        if "msscan" not in n:
            continue
        print(f"| `{_short(n)}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    if args.fetch and args.write:
        fetch = _pmc_per_dispatch(args.fetch, "FETCH_SIZE")
        write = _pmc_per_dispatch(args.write, "WRITE_SIZE")
        copy_kib = COPY_MIB * 1024.0
        cf = [v for k, v in fetch.items() if k == "neg_kernel"]
        cw = [v for k, v in write.items() if k == "neg_kernel"]
        if not cf or not cw:
            raise SystemExit("calibration copy (neg_kernel) not found in the counter runs")
        f_fetch, f_write = copy_kib / cf[0], copy_kib / cw[0]
        print()
        print(f"- copy_fetch_kib: {cf[0]:.0f} (expected {copy_kib:.0f}; factor {f_fetch:.4f})")
        print(f"- copy_write_kib: {cw[0]:.0f} (expected {copy_kib:.0f}; factor {f_write:.4f})")
        print()
        print("| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled MB/dispatch |")
        print("|---|---|---|---|")
        main = None
        for k in sorted(fetch):
            if k == "neg_kernel" or k not in write or not re.search(
                    r"scan_|carry_|bc_prep|step_quads|conv1d_kernel|bwd_main|"
                    r"seg_summaries|bwd_row|reduce_|wide_|copy16|read16", k):
                continue
            mb = (fetch[k] * f_fetch + write[k] * f_write) * 1024 / 1e6
            print(f"| `{k}` | {fetch[k]:.0f} | {write[k]:.0f} | {mb:.2f} |")
            if re.search(MAIN_KERNEL_RE, k):
                main = (fetch[k] * f_fetch + write[k] * f_write) * 1024
        if main is not None:
            print()
            print(f"- traffic_bytes_per_launch: {main:.0f}")
    for dirname in args.counters:
        acc = {}
        for r in _csv(dirname, "counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            if not re.search(r"scan_|carry_|bc_prep|step_quads|bwd_main|bwd_row|seg_summ|conv1d|"
                             r"wide_|reduce_", k):
                continue
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        names = sorted({c for v in acc.values() for c in v})
        print()
        print("| kernel | " + " | ".join(names) + " |")
        print("|---|" + "---|" * len(names))
        for k in sorted(acc):
            vals = [acc[k].get(c) for c in names]
            print(f"| `{k}` | " + " | ".join(f"{sum(v) / len(v):.4g}" if v else "-"
                                             for v in vals) + " |")


# ------------------------------------------------------------------ main --
def measure(ms, w_name, steps, warmup, n_sets, zoh=False, bilinear=False, warm_seconds=0.25):
    import synth
    w = synth.workload(w_name)
    sets = make_sets(w, n_sets)
    t_ms, ph = time_calls(ms, sets, w, steps, warmup, zoh=zoh, bilinear=bilinear,
                          warm_seconds=warm_seconds)
    del sets
    return w, t_ms, ph


def fwd_item(ms, w_name, disc, steps, warmup, n_sets, warm_seconds):
    """One forward line item: call time, rates and kernel times."""
    import synth
    w, t_ms, ph = measure(ms, w_name, steps, warmup, n_sets, zoh=disc == "zoh",
                          bilinear=disc == "bilinear", warm_seconds=warm_seconds)
    e = w.batch * w.L * w.Dn
    opsel = valu_ops_per_element(w.N, disc, softplus=w.softplus)
    main_ms = ph["main"]["mean_ms"]
    item = {"workload": f"{WORKLOAD_TITLE[w.name]} (B{w.batch} L{w.L} D{w.Dn} N{w.N} {w.io}, "
                        f"{disc})",
            "ms_per_call": t_ms, "elem_per_s": e / (t_ms * 1e-3),
            "hbm_gbps": synth.algorithmic_bytes(w) / (t_ms * 1e-3) / 1e9,
            "hbm_frac": synth.algorithmic_bytes(w) / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "ops_per_element": opsel,
            "call_valu_frac": opsel * e / (t_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS,
            "main_valu_frac": opsel * e / (main_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS,
            "kernels_ms": {k: v["per_call_ms"] for k, v in ph.items()
                           if k != "calls" and v["launches"]}}
    return w, t_ms, ph, item


def measure_rates():
    """Chip rates from libmsprobe: v_exp_f32 and fp32 FMA issue (lane
    operations per second, 8 independent chains per lane, 2048 workgroups of
    256 threads), and copy / read bandwidth over 1 GiB (bytes moved per
    second).  Each is the best of 3 timed launches after one warm launch."""
    import ctypes
    import torch
    from selective_state_space_81_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.msprobe_exp.argtypes = [vp, i32, i32, vp]
    lib.msprobe_fma.argtypes = [vp, i32, i32, vp]
    lib.msprobe_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.msprobe_read.argtypes = [vp, vp, i64, i32, vp]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            rc = fn()
            s1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
            ts.append(s0.elapsed_time(s1) * 1e-3)
        return min(ts)

    blocks, iters = 2048, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    lane_ops = blocks * 256 * 8 * iters
    t_exp = best(lambda: lib.msprobe_exp(out.data_ptr(), iters, blocks, sp))
    t_fma = best(lambda: lib.msprobe_fma(out.data_ptr(), iters, blocks, sp))
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    words = nbytes // 16
    cblocks = 16384
    acc = torch.empty(cblocks * 256, dtype=torch.int32, device="cuda")
    t_copy = best(lambda: lib.msprobe_copy(src.data_ptr(), dst.data_ptr(), words, cblocks, sp))
    t_read = best(lambda: lib.msprobe_read(src.data_ptr(), acc.data_ptr(), words, cblocks, sp))
    del src, dst, acc, out
    torch.cuda.empty_cache()
    return {"exp_lane_ops_per_s": lane_ops / t_exp, "fma_lane_ops_per_s": lane_ops / t_fma,
            "exp_vs_fma": t_fma / t_exp,
            "copy_gbps": 2 * nbytes / t_copy / 1e9, "read_gbps": nbytes / t_read / 1e9,
            "valu_peak_lane_ops_per_s": VALU_PEAK_TOPS * 1e12,
            "method": "libmsprobe: 8 independent v_exp_f32 / v_fma_f32 chains per lane, "
                      "2048 x 256 threads x 4096 steps; copy (one contiguous chunk per "
                      "workgroup, 16384 workgroups) and read of 1 GiB with 16-byte "
                      "non-temporal accesses; best of 3"}


def main():
    args = parse()
    if args.rocprof_summary:
        rocprof_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this scan has no multi-GPU path "
              f"(got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_81_amd as ms
    import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ms.load()
    if args.copy_calibration:
        copy_calibration()
    n_sets = args.buffer_sets if args.workload != "long" else 1  # long: 13 GB per set
    if args.zoh and args.bilinear:
        print("--zoh and --bilinear are exclusive", file=sys.stderr)
        sys.exit(2)
    w, t_ms, ph = measure(ms, args.workload, args.steps, args.warmup, n_sets, zoh=args.zoh,
                          bilinear=args.bilinear, warm_seconds=args.warm_seconds)
    disc = "zoh" if args.zoh else ("bilinear" if args.bilinear else "euler")
    torch.cuda.empty_cache()
    elems = w.batch * w.L * w.Dn
    alg_bytes = synth.algorithmic_bytes(w)
    main_ms = ph["main"]["mean_ms"]
    opsel = valu_ops_per_element(w.N, disc, softplus=w.softplus)
    ops = opsel * elems
    achieved = ops / (main_ms * 1e-3) / 1e12
    src = source_hash()
    gbps = alg_bytes / (t_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": elems / (t_ms * 1e-3),
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"f32 compute, {w.io} io",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TITLE[w.name],
                   "batch": w.batch, "seq_len": w.L, "d_inner": w.Dn, "d_state": w.N,
                   "io": w.io, "state": "f32",
                   "discretisation": disc,
                   "softplus_bias": w.softplus, "z_gate": True, "D_skip": True,
                   "buffer_sets": n_sets, "parallelism": "single-gpu"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TOPS,
                     "unit": "TOP/s", "frac": achieved / VALU_PEAK_TOPS,
                     "traffic": load_traffic(w.name, src),
                     "kernel": "scan main pass (writes y)",
                     "kernel_mean_ms": main_ms,
                     "ops_per_element": opsel,
                     "ops_per_launch": ops,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "hbm": {"achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS, "scope": "whole ms_scan_fwd call",
                "algorithmic_bytes_per_call": alg_bytes},
        "call_valu_frac": ops / (t_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS,
        "kernels_ms": {k: v["per_call_ms"] for k, v in ph.items() if k != "calls" and v["launches"]},
        "source_hash": src,
    }
    secondary = not args.no_secondary and args.workload == "m130m" and disc == "euler"
    if secondary:
        rates = measure_rates()
        out["rates"] = rates
        out["hbm"]["frac_of_measured_copy"] = gbps / rates["copy_gbps"]
        items = []
        for d in ("euler", "zoh", "bilinear"):
            _, _, _, it = fwd_item(ms, "m3b", d, max(4, args.steps // 4), 3, 2,
                                   args.warm_seconds)
            items.append(it)
            torch.cuda.empty_cache()
        out["secondary"] = items[0]
        out["m3b_zoh"] = items[1]
        out["m3b_bilinear"] = items[2]
        wl, _, phl, it = fwd_item(ms, "long", "euler", 3, 1, 1, 0.0)
        exps = wl.batch * wl.L * wl.Dn * wl.N
        it["exps_per_call"] = exps
        it["main_exp_per_s"] = exps / (phl["main"]["mean_ms"] * 1e-3)
        it["main_exp_frac_of_measured_rate"] = it["main_exp_per_s"] / rates["exp_lane_ops_per_s"]
        it["call_exp_per_s"] = exps / (it["ms_per_call"] * 1e-3)
        out["long"] = it
        torch.cuda.empty_cache()
        _, _, _, out["wide128_euler"] = fwd_item(ms, "wide128", "euler", 5, 2, 2, args.warm_seconds)
        torch.cuda.empty_cache()
        _, _, _, out["wide64_zoh"] = fwd_item(ms, "wide64", "zoh", 5, 2, 2, args.warm_seconds)
        torch.cuda.empty_cache()
        out["decode"] = measure_decode(ms)
        out["decode"]["frac_of_measured_copy"] = out["decode"]["hbm_gbps"] / rates["copy_gbps"]
        torch.cuda.empty_cache()
        out["conv1d"] = measure_conv(ms)
        out["conv1d"]["frac_of_measured_copy"] = out["conv1d"]["hbm_gbps"] / rates["copy_gbps"]
        torch.cuda.empty_cache()
        out["backward"] = measure_bwd(ms)
        torch.cuda.empty_cache()
        out["dtproj"] = measure_dtproj(ms)
        torch.cuda.empty_cache()
        # d_model 768 for d_inner 1536: rank ceil(768 / 16) = 48
        out["dtproj_wide128"] = measure_dtproj(ms, "wide128", rank=48, reps=10)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, disc)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
