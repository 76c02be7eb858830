"""Seeded synthetic inputs for the selective scan (S6).

This module is shared by the HIP path's tests and bench and by the oracle's
tests.  It only draws and shapes random numbers; it contains none of the
scan's arithmetic.  (The inverse softplus used to place the step size in a
chosen range is a property of the inputs, not a step of the method.)

Every tensor has its own torch.Generator seeded from (seed, workload name,
tensor name), so adding or dropping a tensor never shifts another's stream.
The same call on the same device and torch build gives the same bytes.

Workloads (shapes from the pages' model configurations; value ranges from the
pages' initialisation advice; each recipe is listed in full below):

  tiny      batch 1, L 256, d_inner 64, d_state 16, all fp32.
            A[d,n] = -(n+1); u, B, C, z, D ~ N(0,1);
            delta_raw = softplus^-1(log-uniform[1e-3, 1e-1]); bias = zeros.
  m130m     Mamba-130M layer: batch 8, L 2048, d_inner 1536, d_state 16, bf16.
            A[d,n] = -exp(3n/15); bias[d] = softplus^-1(log-uniform[1e-3,1e-1]);
            delta_raw ~ N(0, 0.5^2); u, B, C, z ~ N(0,1); D ~ N(0,1).
  m3b       Mamba-3B layer: batch 4, L 8192, d_inner 5120, d_state 16, bf16,
            value distributions as ``tiny``.
  long      batch 1, L 1,048,576, d_inner 1536, d_state 64, bf16.
            A[d,n] = -exp(4n/63); delta itself log-uniform[1e-3, 1e-1]
            (softplus off, no bias); u, B, C, z, D ~ N(0,1).
  wide128   batch 2, L 8192, d_inner 1536, d_state 128, bf16, value
            distributions as ``tiny`` (the pages' d_state 64-128 advice for long
            inputs, at a length the whole layer fits in a few hundred MB).
  wide64    as ``wide128`` with d_state 64.
  decode    recurrent decode: batch 256, d_inner 5120, d_state 16; h ~ N(0,1)
            fp32; per step x, delta_raw, B, C, z drawn as ``tiny`` in bf16.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

LOG_LO = math.log(1e-3)
LOG_HI = math.log(1e-1)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    L: int
    Dn: int
    N: int
    io: str                 # "f32" or "bf16"
    a_init: str             # "neg_n1" | "neg_exp3" | "neg_exp4"
    delta_mode: str         # "spinv_logu" | "normal05_bias" | "logu_direct"
    softplus: bool
    discretisations: tuple  # subset of ("euler", "zoh")
    steps: int = 0          # decode steps (decode workload only)
    note: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 256, 64, 16, "f32", "neg_n1", "spinv_logu", True,
                     ("euler", "zoh")),
    "m130m": Workload("m130m", 8, 2048, 1536, 16, "bf16", "neg_exp3", "normal05_bias", True,
                      ("euler",)),
    "m3b": Workload("m3b", 4, 8192, 5120, 16, "bf16", "neg_n1", "spinv_logu", True,
                    ("euler", "zoh")),
    "long": Workload("long", 1, 1 << 20, 1536, 64, "bf16", "neg_exp4", "logu_direct", False,
                     ("euler",)),
    "wide128": Workload("wide128", 2, 8192, 1536, 128, "bf16", "neg_n1", "spinv_logu", True,
                        ("euler", "zoh")),
    "wide64": Workload("wide64", 2, 8192, 1536, 64, "bf16", "neg_n1", "spinv_logu", True,
                       ("euler", "zoh")),
    "decode": Workload("decode", 256, 1, 5120, 16, "bf16", "neg_n1", "spinv_logu", True,
                       ("euler", "zoh"), steps=64),
}


def workload(name: str, **over) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **over) if over else w


def _gen(seed: int, wname: str, tname: str, device) -> torch.Generator:
    h = hashlib.sha256(f"{seed}/{wname}/{tname}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def io_dtype(io: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[io]


def _normal(shape, g, device, std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std) if std != 1.0 else t


def _logu(shape, g, device) -> torch.Tensor:
    """exp(U(ln 1e-3, ln 1e-1)) in float32."""
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(LOG_HI - LOG_LO).add_(LOG_LO).exp_()


def softplus_inverse(x: torch.Tensor) -> torch.Tensor:
    """log(e^x - 1): places softplus(result) at x.  Computed in float64."""
    xd = x.double()
    return torch.log(torch.expm1(xd)).to(x.dtype)


def a_matrix(w: Workload, device="cpu") -> torch.Tensor:
    n = torch.arange(w.N, dtype=torch.float64)
    if w.a_init == "neg_n1":          # A = -(n+1): A_log = log(1..N) init
        row = -(n + 1.0)
    elif w.a_init == "neg_exp3":      # A = -exp(linspace(0, 3, N))
        row = -torch.exp(torch.linspace(0.0, 3.0, w.N, dtype=torch.float64))
    elif w.a_init == "neg_exp4":      # A = -exp(linspace(0, 4, N))
        row = -torch.exp(torch.linspace(0.0, 4.0, w.N, dtype=torch.float64))
    else:
        raise ValueError(w.a_init)
    return row.to(torch.float32).expand(w.Dn, w.N).contiguous().to(device)


def _delta(w: Workload, shape, g, device) -> torch.Tensor:
    if w.delta_mode == "spinv_logu":
        return softplus_inverse(_logu(shape, g, device))
    if w.delta_mode == "normal05_bias":
        return _normal(shape, g, device, std=0.5)
    if w.delta_mode == "logu_direct":
        return _logu(shape, g, device)
    raise ValueError(w.delta_mode)


def _bias(w: Workload, device, seed: int) -> Optional[torch.Tensor]:
    if w.delta_mode == "normal05_bias":
        g = _gen(seed, w.name, "delta_bias", device)
        return softplus_inverse(_logu((w.Dn,), g, device))
    if w.delta_mode == "spinv_logu":
        return torch.zeros(w.Dn, dtype=torch.float32, device=device)
    return None


def scan_inputs(w: Workload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of one full-sequence scan, on ``device``, in the workload's io
    dtype (u, delta, z, B, C) and fp32 (A, D, delta_bias)."""
    dt = io_dtype(w.io)
    x3 = (w.batch, w.L, w.Dn)
    bc = (w.batch, w.L, w.N)

    def g(name):
        return _gen(seed, w.name, name, device)

    out = {
        "u": _normal(x3, g("u"), device).to(dt),
        "delta": _delta(w, x3, g("delta"), device).to(dt),
        "z": _normal(x3, g("z"), device).to(dt),
        "B": _normal(bc, g("B"), device).to(dt),
        "C": _normal(bc, g("C"), device).to(dt),
        "A": a_matrix(w, device),
        "D": _normal((w.Dn,), g("D"), device),
    }
    b = _bias(w, device, seed)
    if b is not None:
        out["delta_bias"] = b
    return out


def decode_inputs(w: Workload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of ``w.steps`` back-to-back decode steps: h0 [batch, Dn, N] fp32
    and per-step x, delta, z [steps, batch, Dn], B, C [steps, batch, N]."""
    dt = io_dtype(w.io)
    s = max(1, w.steps)
    x3 = (s, w.batch, w.Dn)
    bc = (s, w.batch, w.N)

    def g(name):
        return _gen(seed, w.name, name, device)

    out = {
        "h0": _normal((w.batch, w.Dn, w.N), g("h0"), device),
        "x": _normal(x3, g("x"), device).to(dt),
        "delta": _delta(w, x3, g("delta"), device).to(dt),
        "z": _normal(x3, g("z"), device).to(dt),
        "B": _normal(bc, g("B"), device).to(dt),
        "C": _normal(bc, g("C"), device).to(dt),
        "A": a_matrix(w, device),
        "D": _normal((w.Dn,), g("D"), device),
    }
    b = _bias(w, device, seed)
    if b is not None:
        out["delta_bias"] = b
    return out


def conv_inputs(w: Workload, width: int = 4, device="cpu", seed: int = 0,
                history: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of the causal depthwise conv1d that produces the scan input:
    x [batch, L, Dn] ~ N(0,1) (io dtype), weight [Dn, width] ~ N(0, 0.5^2),
    bias [Dn] ~ N(0, 0.1^2) (fp32), and with history=True x_prev
    [batch, width-1, Dn] ~ N(0,1) (io dtype)."""
    dt = io_dtype(w.io)

    def g(name):
        return _gen(seed, w.name, "conv_" + name, device)

    out = {
        "x": _normal((w.batch, w.L, w.Dn), g("x"), device).to(dt),
        "weight": _normal((w.Dn, width), g("weight"), device, std=0.5),
        "bias": _normal((w.Dn,), g("bias"), device, std=0.1),
    }
    if history and width > 1:
        out["x_prev"] = _normal((w.batch, width - 1, w.Dn), g("x_prev"), device).to(dt)
    return out


def dtproj_inputs(w: Workload, rank: int, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of the fused low-rank step projection: dt_low [batch, L, rank]
    ~ N(0,1) and W_dt [Dn, rank] ~ N(0, 0.5^2 / rank), both in the io dtype,
    so the projected raw step has standard deviation about 0.5 (the spread of
    the 130M-layer workload's raw step)."""
    dt = io_dtype(w.io)

    def g(name):
        return _gen(seed, w.name, "dtproj_" + name, device)

    return {
        "dt_low": _normal((w.batch, w.L, rank), g("dt_low"), device).to(dt),
        "W_dt": _normal((w.Dn, rank), g("W_dt"), device, std=0.5 / rank ** 0.5).to(dt),
    }


def algorithmic_bytes(w: Workload) -> int:
    """Bytes the scan must move once: u, delta, z read and y written
    ([batch, L, Dn] each, io dtype), B and C read ([batch, L, N]), A read
    ([Dn, N] fp32), D and delta_bias read ([Dn] fp32 each)."""
    e = 2 if w.io == "bf16" else 4
    return (4 * w.batch * w.L * w.Dn * e + 2 * w.batch * w.L * w.N * e
            + w.Dn * w.N * 4 + 2 * w.Dn * 4)
