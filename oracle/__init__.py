"""fp64 CPU oracle for the selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and this package imports nothing from the HIP library.

The arithmetic lives in ``msscan_oracle.c`` (plain C, double precision, OpenMP
over independent channels).  This module only converts numpy/torch arrays to
contiguous float64 and calls it through ctypes.  See the C file's header for
the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_scan.argtypes = [dp] * 9 + [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                               dp, dp, ctypes.c_int]
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_step.argtypes = [dp] * 9 + [ctypes.c_int, ctypes.c_int, i64, i64, i64, dp]
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [dp] * 9 + [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64] \
            + [dp] * 11 + [ctypes.c_int]
        lib.oracle_conv1d.restype = ctypes.c_int
        lib.oracle_conv1d.argtypes = [dp] * 4 + [i64, ctypes.c_int, i64, i64, i64, dp,
                                                 ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: exact widening on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _disc(zoh: bool, bilinear: bool) -> int:
    if zoh and bilinear:
        raise ValueError("zoh and bilinear are exclusive")
    return 2 if bilinear else (1 if zoh else 0)


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
         softplus: bool = True, zoh: bool = False, nthreads: int = 0, bilinear: bool = False
         ) -> Tuple[np.ndarray, np.ndarray]:
    """Selective scan in fp64 (Euler by default; zoh or bilinear pick the
    other discretisations).

    u, delta, z: [batch, L, Dn]; B, C: [batch, L, N]; A: [Dn, N];
    D, delta_bias: [Dn]; h0: [batch, Dn, N].  Returns (y [batch, L, Dn],
    h_last [batch, Dn, N]) as float64 arrays.
    """
    lib = _load()
    u, delta, A, B, C = (_f64(t) for t in (u, delta, A, B, C))
    D, z, delta_bias, h0 = (_f64(t) for t in (D, z, delta_bias, h0))
    batch, L, Dn = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (Dn, N)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    assert D is None or D.shape == (Dn,)
    assert delta_bias is None or delta_bias.shape == (Dn,)
    assert h0 is None or h0.shape == (batch, Dn, N)
    y = np.empty((batch, L, Dn), dtype=np.float64)
    h_last = np.empty((batch, Dn, N), dtype=np.float64)
    rc = lib.oracle_scan(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(delta_bias), _ptr(h0), int(bool(softplus)), _disc(zoh, bilinear),
                         batch, L, Dn, N, _ptr(y), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_scan failed with code {rc}")
    return y, h_last


def scan_dtproj(u, dt_low, W_dt, A, B, C, D=None, z=None, delta_bias=None, h0=None,
                softplus: bool = True, zoh: bool = False, nthreads: int = 0,
                bilinear: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """The scan with its raw step given as a low-rank projection, in fp64.

    The step size is softplus of a linear map of the input plus a bias (jsqmd
    page, section 2.2); in the block, x_proj yields a narrow dt slice per
    timestep that dt_proj lifts to d_inner (lmnt page, section 3.2).  So
        delta[b, t, d] = sum_r W_dt[d, r] * dt_low[b, t, r]
    (a matrix product, numpy's, in fp64 with no rounding to the io type), and
    then exactly ``scan`` with that delta.

    dt_low: [batch, L, rank]; W_dt: [Dn, rank] (a linear layer's out x in
    weight); the rest as for ``scan``.  Returns (y, h_last)."""
    dt_low, W_dt = _f64(dt_low), _f64(W_dt)
    assert dt_low.ndim == 3 and W_dt.ndim == 2 and dt_low.shape[2] == W_dt.shape[1]
    delta = np.matmul(dt_low, W_dt.T)
    return scan(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias, h0=h0, softplus=softplus,
                zoh=zoh, nthreads=nthreads, bilinear=bilinear)


def step(h, x, delta, A, B, C, D=None, z=None, delta_bias=None,
         softplus: bool = True, zoh: bool = False, bilinear: bool = False
         ) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step in fp64.  h: [batch, Dn, N] (not modified; the updated
    state is returned); x, delta, z: [batch, Dn]; B, C: [batch, N].
    Returns (y [batch, Dn], h_new [batch, Dn, N])."""
    lib = _load()
    h = _f64(h).copy()
    x, delta, A, B, C = (_f64(t) for t in (x, delta, A, B, C))
    D, z, delta_bias = (_f64(t) for t in (D, z, delta_bias))
    batch, Dn = x.shape
    N = A.shape[1]
    assert h.shape == (batch, Dn, N) and B.shape == (batch, N) and C.shape == (batch, N)
    y = np.empty((batch, Dn), dtype=np.float64)
    rc = lib.oracle_step(_ptr(h), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                         _ptr(z), _ptr(delta_bias), int(bool(softplus)), _disc(zoh, bilinear),
                         batch, Dn, N, _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_step failed with code {rc}")
    return y, h


def conv1d(x, w, bias=None, x_prev=None, silu: bool = True, nthreads: int = 0) -> np.ndarray:
    """Causal depthwise conv1d (+ silu) in fp64.

    x: [batch, L, Dn]; w: [Dn, width]; bias: [Dn]; x_prev: [batch, width-1, Dn]
    (the inputs before t = 0, oldest first; None = zeros).  Returns u
    [batch, L, Dn] as float64."""
    xf, wf, bf, pf = _f64(x), _f64(w), _f64(bias), _f64(x_prev)
    batch, L, Dn = xf.shape
    width = wf.shape[1]
    assert wf.shape == (Dn, width)
    if bf is not None:
        assert bf.shape == (Dn,)
    if pf is not None:
        assert pf.shape == (batch, width - 1, Dn)
    u = np.empty((batch, L, Dn), dtype=np.float64)
    rc = _load().oracle_conv1d(_ptr(xf), _ptr(wf), _ptr(bf), _ptr(pf), width, int(silu),
                               batch, L, Dn, _ptr(u), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_conv1d failed ({rc})")
    return u


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, h0=None, dh_last=None,
             softplus: bool = True, zoh: bool = False, bilinear: bool = False,
             nthreads: int = 0) -> dict:
    """Gradients of scan() in fp64: given dy [batch, L, Dn] (and optionally
    dh_last [batch, Dn, N]), returns a dict with du, ddelta (w.r.t. the raw
    delta), dA, dB, dC, and dz / dD / dbias / dh0 (dbias and dh0 always; dz
    and dD when z and D are given)."""
    lib = _load()
    u, delta, A, B, C, dy = (_f64(t) for t in (u, delta, A, B, C, dy))
    D, z, delta_bias, h0, dh_last = (_f64(t) for t in (D, z, delta_bias, h0, dh_last))
    batch, L, Dn = u.shape
    N = A.shape[1]
    assert dy.shape == u.shape
    out = {"du": np.empty_like(u), "ddelta": np.empty_like(u), "dA": np.empty((Dn, N)),
           "dB": np.empty((batch, L, N)), "dC": np.empty((batch, L, N)),
           "dbias": np.empty(Dn), "dh0": np.empty((batch, Dn, N))}
    out["dz"] = np.empty_like(u) if z is not None else None
    out["dD"] = np.empty(Dn) if D is not None else None
    rc = lib.oracle_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), _ptr(h0), int(bool(softplus)),
                             _disc(zoh, bilinear), batch, L, Dn, N, _ptr(dy), _ptr(dh_last),
                             _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
                             _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                             _ptr(out["dbias"]), _ptr(out["dh0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_scan_bwd failed with code {rc}")
    return out
