"""Python binding of libmsscan (selective scan, S6, on MI355X / gfx950).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libmsscan.so`` behind the C ABI declared in ``include/msscan.h``.  Torch is
used for device memory and streams: tensors are passed as raw device pointers
together with the current HIP stream.  There is no CPU fallback -- if the
library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsscan.so")

MS_OK = 0
MS_F32 = 0
MS_BF16 = 1
MS_SOFTPLUS = 1
MS_ZOH = 2
MS_BILINEAR = 4

STATUS = {0: "MS_OK", 1: "MS_ERR_NULL", 2: "MS_ERR_SHAPE", 3: "MS_ERR_DTYPE",
          4: "MS_ERR_FLAGS", 5: "MS_ERR_ALIGN", 6: "MS_ERR_WORKSPACE",
          7: "MS_ERR_UNSUPPORTED", 8: "MS_ERR_HIP"}

EXPORTS = ("ms_scan_workspace_bytes", "ms_scan_fwd", "ms_state_update", "ms_status_string",
           "ms_last_error", "ms_abi_version", "ms_profile_begin", "ms_profile_end",
           "ms_conv1d_silu", "ms_scan_bwd_workspace_bytes", "ms_scan_bwd",
           "ms_scan_fwd_dtproj", "ms_scan_dtproj_workspace_bytes", "ms_scan_fwd_noalloc",
           "ms_scan_checkpoint_bytes", "ms_scan_fwd_checkpoint",
           "ms_scan_bwd_checkpoint_workspace_bytes", "ms_scan_bwd_checkpoint")

PHASES = ("prep", "summary", "carry", "main", "step", "conv", "reduce")  # ms_phase order


class MsDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("io", ctypes.c_int32)]


class MsProfile(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int32), ("launches", ctypes.c_int32 * len(PHASES)),
                ("total_ms", ctypes.c_double * len(PHASES))]


class MsError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load(path: Optional[str] = None):
    """Load libmsscan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime; importing it first makes this library
    # bind to that same runtime (one device context per process) rather than
    # loading a second copy from the ROCm install.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m selective_state_space_81_amd.build`")
    lib = ctypes.CDLL(p)
    vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int32
    lib.ms_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ms_scan_workspace_bytes.argtypes = [ctypes.POINTER(MsDims), u32]
    lib.ms_scan_fwd.restype = ctypes.c_int
    lib.ms_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, vp, vp,
                                ctypes.POINTER(MsDims), vp, ctypes.c_size_t, vp]
    lib.ms_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ms_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, vp, vp,
                                        ctypes.POINTER(MsDims), vp]
    lib.ms_scan_dtproj_workspace_bytes.restype = ctypes.c_size_t
    lib.ms_scan_dtproj_workspace_bytes.argtypes = [ctypes.POINTER(MsDims), u32]
    lib.ms_scan_fwd_dtproj.restype = ctypes.c_int
    lib.ms_scan_fwd_dtproj.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, u32, vp, vp, vp,
                                       ctypes.POINTER(MsDims), vp, ctypes.c_size_t, vp]
    lib.ms_state_update.restype = ctypes.c_int
    lib.ms_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp,
                                    i32, i32, i32, i32, vp]
    lib.ms_status_string.restype = ctypes.c_char_p
    lib.ms_status_string.argtypes = [ctypes.c_int]
    lib.ms_last_error.restype = ctypes.c_char_p
    lib.ms_last_error.argtypes = []
    lib.ms_abi_version.restype = ctypes.c_int
    lib.ms_abi_version.argtypes = []
    lib.ms_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ms_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(MsDims), u32]
    lib.ms_scan_bwd.restype = ctypes.c_int
    lib.ms_scan_bwd.argtypes = [vp] * 8 + [u32] + [vp] * 12 + [ctypes.POINTER(MsDims), vp,
                                                                ctypes.c_size_t, vp]
    lib.ms_scan_checkpoint_bytes.argtypes = [ctypes.POINTER(MsDims), u32]
    lib.ms_scan_checkpoint_bytes.restype = ctypes.c_size_t
    lib.ms_scan_fwd_checkpoint.argtypes = [vp] * 8 + [u32] + [vp] * 4 + [ctypes.POINTER(MsDims),
                                                                          vp]
    lib.ms_scan_fwd_checkpoint.restype = ctypes.c_int
    lib.ms_scan_bwd_checkpoint_workspace_bytes.argtypes = [ctypes.POINTER(MsDims), u32]
    lib.ms_scan_bwd_checkpoint_workspace_bytes.restype = ctypes.c_size_t
    lib.ms_scan_bwd_checkpoint.argtypes = [vp] * 8 + [u32] + [vp] * 12 + [
        ctypes.POINTER(MsDims), vp, ctypes.c_size_t, vp]
    lib.ms_scan_bwd_checkpoint.restype = ctypes.c_int
    lib.ms_conv1d_silu.restype = ctypes.c_int
    lib.ms_conv1d_silu.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, ctypes.c_int64, i32, i32,
                                   vp]
    lib.ms_profile_begin.restype = ctypes.c_int
    lib.ms_profile_begin.argtypes = [i32]
    lib.ms_profile_end.restype = ctypes.c_int
    lib.ms_profile_end.argtypes = [ctypes.POINTER(MsProfile)]
    if path is None:
        _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _io(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MS_BF16
    if t.dtype == torch.float32:
        return MS_F32
    raise TypeError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _chk(t, name: str, dtype, shape) -> None:
    """The layout include/msscan.h specifies for a tensor argument: a
    contiguous device tensor of this dtype and shape (None passes: the
    argument is optional).  Raises before anything reaches the library."""
    if t is None:
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device (GPU) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _chk_scan(u, delta, A, B, C, D, z, delta_bias, h0=None, h_last=None, y=None):
    """Checks of the forward scan's arguments; returns (batch, L, Dn, N, io dtype)."""
    import torch
    if not getattr(u, "is_cuda", False) or u.dim() != 3:
        raise ValueError("u must be a [batch, L, d_inner] device tensor")
    _io(u)
    batch, L, Dn = u.shape
    if A is None or A.dim() != 2:
        raise ValueError("A must be a [d_inner, d_state] tensor")
    N = A.shape[1]
    io, f32 = u.dtype, torch.float32
    _chk(u, "u", io, (batch, L, Dn))
    _chk(delta, "delta", io, (batch, L, Dn))
    _chk(A, "A", f32, (Dn, N))
    _chk(B, "B", io, (batch, L, N))
    _chk(C, "C", io, (batch, L, N))
    _chk(D, "D", f32, (Dn,))
    _chk(z, "z", io, (batch, L, Dn))
    _chk(delta_bias, "delta_bias", f32, (Dn,))
    _chk(h0, "h0", f32, (batch, Dn, N))
    _chk(h_last, "h_last", f32, (batch, Dn, N))
    _chk(y, "y", io, (batch, L, Dn))
    return batch, L, Dn, N, io


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int):
    if rc != MS_OK:
        raise MsError(rc, load().ms_last_error().decode())


def flags(softplus: bool = True, zoh: bool = False, bilinear: bool = False) -> int:
    return (MS_SOFTPLUS if softplus else 0) | (MS_ZOH if zoh else 0) | \
        (MS_BILINEAR if bilinear else 0)


def dims(batch: int, seqlen: int, d_inner: int, d_state: int, io: int) -> MsDims:
    return MsDims(batch, seqlen, d_inner, d_state, io)


def workspace_bytes(batch: int, seqlen: int, d_inner: int, d_state: int, io: int,
                    flag_bits: int = MS_SOFTPLUS) -> int:
    d = dims(batch, seqlen, d_inner, d_state, io)
    n = load().ms_scan_workspace_bytes(ctypes.byref(d), flag_bits)
    if n == ctypes.c_size_t(-1).value:
        raise MsError(2, "invalid dims")
    return int(n)


def dtproj_workspace_bytes(batch: int, seqlen: int, d_inner: int, d_state: int, io: int,
                           flag_bits: int = MS_SOFTPLUS) -> int:
    """ms_scan_dtproj_workspace_bytes: workspace of ms_scan_fwd_dtproj."""
    d = dims(batch, seqlen, d_inner, d_state, io)
    n = load().ms_scan_dtproj_workspace_bytes(ctypes.byref(d), flag_bits)
    if n == ctypes.c_size_t(-1).value:
        raise MsError(2, "invalid dims")
    return int(n)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, softplus=True, zoh=False,
             y=None, h0=None, h_last=None, workspace=None, stream=None, bilinear=False):
    """ms_scan_fwd on torch device tensors.  Allocates y (and the workspace)
    when not given -- that allocation is torch's, outside the library.
    Returns y."""
    import torch
    batch, L, Dn, N, _ = _chk_scan(u, delta, A, B, C, D, z, delta_bias, h0, h_last, y)
    io = _io(u)
    fl = flags(softplus, zoh, bilinear)
    if y is None:
        y = torch.empty_like(u)
    ws_n = workspace_bytes(batch, L, Dn, N, io, fl)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=u.device)
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    d = dims(batch, L, Dn, N, io)
    rc = load().ms_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(delta_bias), fl, _ptr(y), _ptr(h0), _ptr(h_last),
                            ctypes.byref(d), _ptr(workspace), ws_size, _stream(stream))
    _check(rc)
    return y


NOALLOC_MAX_BYTES = 64 << 20  # MS_NOALLOC_MAX_BYTES


def scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, softplus=True,
                     zoh=False, bilinear=False, y, h0=None, h_last=None, stream=None):
    """ms_scan_fwd_noalloc on torch device tensors: the forward scan with the
    library's own device scratch (no workspace argument).  y must be given
    (nothing is allocated here either).  Returns y."""
    batch, L, Dn, N, _ = _chk_scan(u, delta, A, B, C, D, z, delta_bias, h0, h_last, y)
    if y is None:
        raise ValueError("y is required (scan_fwd_noalloc allocates nothing)")
    d = dims(batch, L, Dn, N, _io(u))
    rc = load().ms_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(delta_bias), flags(softplus, zoh, bilinear),
                                    _ptr(y), _ptr(h0), _ptr(h_last), ctypes.byref(d),
                                    _stream(stream))
    _check(rc)
    return y


def scan_fwd_dtproj(u, dt_low, W_dt, A, B, C, D=None, z=None, delta_bias=None, *,
                    softplus=True, zoh=False, bilinear=False, y=None, h0=None, h_last=None,
                    workspace=None, stream=None):
    """ms_scan_fwd_dtproj on torch device tensors: the scan with its raw step
    projected from dt_low [batch][L][rank] by W_dt [d_inner][rank] inside the
    kernel.  Allocates y (and the workspace) when not given.  Returns y."""
    import torch
    batch, L, Dn, N, iod = _chk_scan(u, u, A, B, C, D, z, delta_bias, h0, h_last, y)
    if W_dt is None or W_dt.dim() != 2:
        raise ValueError("W_dt must be a [d_inner, rank] tensor")
    rank = int(W_dt.shape[1])
    _chk(dt_low, "dt_low", iod, (batch, L, rank))
    _chk(W_dt, "W_dt", iod, (Dn, rank))
    io = _io(u)
    fl = flags(softplus, zoh, bilinear)
    if y is None:
        y = torch.empty_like(u)
    ws_n = dtproj_workspace_bytes(batch, L, Dn, N, io, fl)
    if workspace is None and ws_n:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=u.device)
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    d = dims(batch, L, Dn, N, io)
    rc = load().ms_scan_fwd_dtproj(_ptr(u), _ptr(dt_low), _ptr(W_dt), rank, _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), fl, _ptr(y),
                                   _ptr(h0), _ptr(h_last), ctypes.byref(d), _ptr(workspace),
                                   ws_size, _stream(stream))
    _check(rc)
    return y


def state_update(h, x_t, delta_t, A, B_t, C_t, D=None, z_t=None, delta_bias=None, *,
                 softplus=True, zoh=False, y_t=None, stream=None, bilinear=False):
    """ms_state_update on torch device tensors; h is updated in place.
    Returns y_t."""
    import torch
    if not getattr(x_t, "is_cuda", False) or x_t.dim() != 2:
        raise ValueError("x_t must be a [batch, d_inner] device tensor")
    _io(x_t)
    batch, Dn = x_t.shape
    if A is None or A.dim() != 2:
        raise ValueError("A must be a [d_inner, d_state] tensor")
    N = A.shape[1]
    io, f32 = x_t.dtype, torch.float32
    _chk(h, "h", f32, (batch, Dn, N))
    _chk(delta_t, "delta_t", io, (batch, Dn))
    _chk(A, "A", f32, (Dn, N))
    _chk(B_t, "B_t", io, (batch, N))
    _chk(C_t, "C_t", io, (batch, N))
    _chk(D, "D", f32, (Dn,))
    _chk(z_t, "z_t", io, (batch, Dn))
    _chk(delta_bias, "delta_bias", f32, (Dn,))
    _chk(y_t, "y_t", io, (batch, Dn))
    if y_t is None:
        y_t = torch.empty_like(x_t)
    rc = load().ms_state_update(_ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t),
                                _ptr(C_t), _ptr(D), _ptr(z_t), _ptr(delta_bias),
                                flags(softplus, zoh, bilinear), _ptr(y_t), batch, Dn, N, _io(x_t),
                                _stream(stream))
    _check(rc)
    return y_t


_scan_fn = None


def _scan_function():
    """torch.autograd.Function over ms_scan_fwd / ms_scan_bwd (built on first
    use, so that importing this package does not import torch)."""
    global _scan_fn
    if _scan_fn is None:
        import torch

        class ScanFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, u, delta, A, B, C, D, z, delta_bias, h0, softplus, zoh, bilinear,
                        save_states):
                kw = dict(D=D, z=z, delta_bias=delta_bias, softplus=softplus, zoh=zoh,
                          bilinear=bilinear, h0=h0)
                ck = None
                if save_states and checkpoint_bytes(*u.shape, B.shape[-1], _io(u),
                                                    flags(softplus, zoh, bilinear)):
                    y, ck = scan_fwd_checkpoint(u, delta, A, B, C, **kw)
                else:
                    y = scan_fwd(u, delta, A, B, C, **kw)
                ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0, ck)
                ctx.disc = (softplus, zoh, bilinear)
                return y

            @staticmethod
            def backward(ctx, dy):
                u, delta, A, B, C, D, z, delta_bias, h0, ck = ctx.saved_tensors
                softplus, zoh, bilinear = ctx.disc
                kw = dict(D=D, z=z, delta_bias=delta_bias, softplus=softplus, zoh=zoh,
                          bilinear=bilinear, want_dh0=h0 is not None and ctx.needs_input_grad[8])
                if ck is not None:
                    g = scan_bwd_checkpoint(u, delta, A, B, C, dy.contiguous(), ck, **kw)
                else:
                    g = scan_bwd(u, delta, A, B, C, dy.contiguous(), h0=h0, **kw)
                return (g["du"], g["ddelta"], g["dA"], g["dB"].to(B.dtype),
                        g["dC"].to(C.dtype), g["dD"], g["dz"],
                        g["dbias"] if delta_bias is not None else None,
                        g["dh0"] if h0 is not None else None, None, None, None, None)

        _scan_fn = ScanFn
    return _scan_fn


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
                   softplus=True, zoh=False, bilinear=False, save_states=True):
    """The scan as a differentiable torch operation: the forward is
    ms_scan_fwd and the backward ms_scan_bwd (gradients of every tensor
    argument; dB and dC are returned in B's and C's dtype).  With save_states,
    where the checkpointed pair serves the dims (ms_scan_checkpoint_bytes > 0)
    the forward is ms_scan_fwd_checkpoint and its block states are kept for
    ms_scan_bwd_checkpoint (4 * d_state / 16 bytes per element) instead of
    being recomputed.  Returns y."""
    return _scan_function().apply(u, delta, A, B, C, D, z, delta_bias, h0, softplus, zoh,
                                  bilinear, save_states)


def profile_begin(max_calls: int) -> None:
    """ms_profile_begin: time the kernels of the next max_calls calls."""
    rc = load().ms_profile_begin(max_calls)
    if rc != MS_OK:
        raise MsError(rc, "ms_profile_begin failed")


def profile_end() -> dict:
    """ms_profile_end: wait for the recorded events and return, per phase,
    the number of timed launches, their mean kernel time (ms per launch) and
    the phase's kernel time per timed call (ms; a call may launch a phase's
    kernel more than once)."""
    out = MsProfile()
    rc = load().ms_profile_end(ctypes.byref(out))
    if rc != MS_OK:
        raise MsError(rc, "ms_profile_end failed")
    res = {"calls": out.calls}
    for i, name in enumerate(PHASES):
        n = out.launches[i]
        res[name] = {"launches": n, "mean_ms": (out.total_ms[i] / n) if n else None,
                     "per_call_ms": (out.total_ms[i] / out.calls) if n else None}
    return res


def conv1d_silu(x, weight, bias=None, x_prev=None, *, silu=True, u=None, stream=None):
    """ms_conv1d_silu on torch device tensors: causal depthwise conv1d of x
    ([batch, L, d_inner]) with weight [d_inner, width] (+ bias), then silu.
    x_prev: [batch, width-1, d_inner] inputs before t = 0 (None = zeros).
    Returns u."""
    import torch
    if not getattr(x, "is_cuda", False) or x.dim() != 3:
        raise ValueError("x must be a [batch, L, d_inner] device tensor")
    _io(x)
    batch, L, Dn = x.shape
    if weight is None or weight.dim() != 2:
        raise ValueError("weight must be a [d_inner, width] tensor")
    width = weight.shape[1]
    _chk(weight, "weight", torch.float32, (Dn, width))
    _chk(bias, "bias", torch.float32, (Dn,))
    if width > 1:
        _chk(x_prev, "x_prev", x.dtype, (batch, width - 1, Dn))
    _chk(u, "u", x.dtype, (batch, L, Dn))
    if u is None:
        u = torch.empty_like(x)
    rc = load().ms_conv1d_silu(_ptr(x), _ptr(weight), _ptr(bias), _ptr(x_prev), width,
                               1 if silu else 0, _ptr(u), batch, L, Dn, _io(x), _stream(stream))
    _check(rc)
    return u


def scan_bwd_workspace_bytes(batch: int, seqlen: int, d_inner: int, d_state: int, io: int,
                             flag_bits: int = MS_SOFTPLUS) -> int:
    d = dims(batch, seqlen, d_inner, d_state, io)
    n = load().ms_scan_bwd_workspace_bytes(ctypes.byref(d), flag_bits)
    if n == ctypes.c_size_t(-1).value:
        raise MsError(2, "invalid dims for ms_scan_bwd")
    return int(n)


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, *, softplus=True,
             zoh=False, bilinear=False, h0=None, dh_last=None, workspace=None, stream=None,
             want_dh0=True):
    """ms_scan_bwd on torch device tensors: gradients of scan_fwd for the
    output gradient dy (and optionally dh_last).  Allocates the outputs (and
    the workspace when not given).  Returns a dict: du, ddelta, dz (io dtype),
    dA, dB, dC, dD, dbias, dh0 (fp32); dz / dD are None when z / D are."""
    import torch
    batch, L, Dn, N, iod = _chk_scan(u, delta, A, B, C, D, z, delta_bias, h0)
    _chk(dy, "dy", iod, (batch, L, Dn))
    _chk(dh_last, "dh_last", torch.float32, (batch, Dn, N))
    io = _io(u)
    fl = flags(softplus, zoh, bilinear)
    dev = u.device
    f32 = torch.float32
    out = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
           "dz": torch.empty_like(u) if z is not None else None,
           "dA": torch.empty(Dn, N, dtype=f32, device=dev),
           "dB": torch.empty(batch, L, N, dtype=f32, device=dev),
           "dC": torch.empty(batch, L, N, dtype=f32, device=dev),
           "dD": torch.empty(Dn, dtype=f32, device=dev) if D is not None else None,
           "dbias": torch.empty(Dn, dtype=f32, device=dev),
           "dh0": torch.empty(batch, Dn, N, dtype=f32, device=dev) if want_dh0 else None}
    ws_n = scan_bwd_workspace_bytes(batch, L, Dn, N, io, fl)
    if workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = workspace.numel() * workspace.element_size()
    d = dims(batch, L, Dn, N, io)
    rc = load().ms_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(delta_bias), fl, _ptr(h0), _ptr(dy), _ptr(dh_last),
                            _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
                            _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                            _ptr(out["dbias"]), _ptr(out["dh0"]), ctypes.byref(d),
                            _ptr(workspace), ws_size, _stream(stream))
    _check(rc)
    return out


def checkpoint_bytes(batch: int, seqlen: int, d_inner: int, d_state: int, io: int,
                     flag_bits: int = MS_SOFTPLUS) -> int:
    """ms_scan_checkpoint_bytes: size of the forward-saved checkpoints (0 when
    the checkpointed pair does not serve these dims)."""
    d = dims(batch, seqlen, d_inner, d_state, io)
    n = load().ms_scan_checkpoint_bytes(ctypes.byref(d), flag_bits)
    if n == ctypes.c_size_t(-1).value:
        raise MsError(2, "invalid dims")
    return int(n)


def scan_fwd_checkpoint(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, softplus=True,
                        zoh=False, bilinear=False, y=None, h0=None, h_last=None,
                        checkpoint=None, stream=None):
    """ms_scan_fwd_checkpoint on torch device tensors: the forward scan that
    also saves the backward's block-state checkpoints.  Allocates y and the
    checkpoint ([batch, ceil(L/16), d_inner, d_state] fp32) when not given.
    Returns (y, checkpoint)."""
    import torch
    batch, L, Dn, N, _ = _chk_scan(u, delta, A, B, C, D, z, delta_bias, h0, h_last, y)
    io = _io(u)
    fl = flags(softplus, zoh, bilinear)
    if checkpoint_bytes(batch, L, Dn, N, io, fl) == 0:
        raise MsError(7, "no forward checkpoints for these dims")
    if y is None:
        y = torch.empty_like(u)
    if checkpoint is None:
        checkpoint = torch.empty(batch, (L + 15) // 16, Dn, N, dtype=torch.float32,
                                 device=u.device)
    _chk(checkpoint, "checkpoint", torch.float32, (batch, (L + 15) // 16, Dn, N))
    d = dims(batch, L, Dn, N, io)
    rc = load().ms_scan_fwd_checkpoint(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(z), _ptr(delta_bias), fl, _ptr(y), _ptr(h0),
                                       _ptr(h_last), _ptr(checkpoint), ctypes.byref(d),
                                       _stream(stream))
    _check(rc)
    return y, checkpoint


def scan_bwd_checkpoint_workspace_bytes(batch: int, seqlen: int, d_inner: int, d_state: int,
                                        io: int, flag_bits: int = MS_SOFTPLUS) -> int:
    d = dims(batch, seqlen, d_inner, d_state, io)
    n = load().ms_scan_bwd_checkpoint_workspace_bytes(ctypes.byref(d), flag_bits)
    if n == ctypes.c_size_t(-1).value:
        raise MsError(7, "no checkpointed backward for these dims")
    return int(n)


def scan_bwd_checkpoint(u, delta, A, B, C, dy, checkpoint, D=None, z=None, delta_bias=None, *,
                        softplus=True, zoh=False, bilinear=False, dh_last=None, workspace=None,
                        stream=None, want_dh0=True):
    """ms_scan_bwd_checkpoint on torch device tensors: scan_bwd with the
    checkpoint that scan_fwd_checkpoint saved (h0 is in it).  Returns the
    dict of scan_bwd."""
    import torch
    batch, L, Dn, N, iod = _chk_scan(u, delta, A, B, C, D, z, delta_bias)
    _chk(dy, "dy", iod, (batch, L, Dn))
    _chk(dh_last, "dh_last", torch.float32, (batch, Dn, N))
    _chk(checkpoint, "checkpoint", torch.float32, (batch, (L + 15) // 16, Dn, N))
    io = _io(u)
    fl = flags(softplus, zoh, bilinear)
    dev = u.device
    f32 = torch.float32
    out = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
           "dz": torch.empty_like(u) if z is not None else None,
           "dA": torch.empty(Dn, N, dtype=f32, device=dev),
           "dB": torch.empty(batch, L, N, dtype=f32, device=dev),
           "dC": torch.empty(batch, L, N, dtype=f32, device=dev),
           "dD": torch.empty(Dn, dtype=f32, device=dev) if D is not None else None,
           "dbias": torch.empty(Dn, dtype=f32, device=dev),
           "dh0": torch.empty(batch, Dn, N, dtype=f32, device=dev) if want_dh0 else None}
    ws_n = scan_bwd_checkpoint_workspace_bytes(batch, L, Dn, N, io, fl)
    if workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = workspace.numel() * workspace.element_size()
    d = dims(batch, L, Dn, N, io)
    rc = load().ms_scan_bwd_checkpoint(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), fl,
        _ptr(checkpoint), _ptr(dy), _ptr(dh_last), _ptr(out["du"]), _ptr(out["ddelta"]),
        _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
        _ptr(out["dbias"]), _ptr(out["dh0"]), ctypes.byref(d), _ptr(workspace), ws_size,
        _stream(stream))
    _check(rc)
    return out
