"""S5 layer forward hot path on AMD MI355X (gfx950): Python binding.

Thin ctypes layer over the C ABI in include/s5.h (libs5.so, built in-tree by
``diagonal_state_space_amd.build_lib``). It only marshals arguments: checks
device, dtype, shape and contiguity of torch tensors, passes their device
pointers and the current HIP stream, and turns status codes into exceptions.
Every step of the computation runs in the library's kernels; PyTorch provides
device memory and streams. There is no fallback: if libs5.so is missing or a
GPU is not present, the calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "S5Error",
    "S5_F32",
    "S5_BF16",
    "S5_MAX_P",
    "S5_MAX_H",
    "lib",
    "lib_path",
    "discretize",
    "forward",
    "forward_timevarying",
    "forward_stateful",
    "forward_timevarying_stateful",
    "set_profiling_events",
    "status_string",
]

S5_F32 = 0
S5_BF16 = 1
S5_MAX_P = 256
S5_MAX_H = 512

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libs5.so")
_lib = None

EXPORTS = ("s5_discretize", "s5_forward", "s5_forward_noalloc", "s5_forward_timevarying", "s5_forward_stateful",
           "s5_forward_timevarying_stateful", "s5_forward_ex", "s5_step", "s5_glu", "s5_status_string",
           "s5_set_profiling_events")

# option bits of s5_forward_ex (include/s5.h)
FLAG_HALF_SPECTRUM = 1 << 0
FLAG_BILINEAR = 1 << 1
FLAG_GELU = 1 << 2
FLAG_BIDIRECTIONAL = 1 << 3
FLAG_GELU_TANH = 1 << 4
FLAG_GLU = 1 << 5


class ForwardDesc(ctypes.Structure):
    """s5_forward_desc of include/s5.h."""
    _fields_ = [("size", ctypes.c_uint32), ("flags", ctypes.c_uint32), ("io", ctypes.c_int),
                ("B", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64), ("P", ctypes.c_int64),
                ("u", ctypes.c_void_p), ("lam", ctypes.c_void_p), ("b_tilde", ctypes.c_void_p),
                ("c_tilde", ctypes.c_void_p), ("d", ctypes.c_void_p), ("log_delta", ctypes.c_void_p),
                ("delta", ctypes.c_void_p), ("x0", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("x_last", ctypes.c_void_p),
                ("glu_w", ctypes.c_void_p), ("glu_bias", ctypes.c_void_p), ("glu_variant", ctypes.c_int32)]


class S5Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libs5.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} not found: build it with "
                              "`python -m diagonal_state_space_amd.build_lib`")
        # torch first: it carries its own HIP runtime, and libs5.so must bind
        # to that one (loaded before torch, it would bind to the system's, and
        # torch's streams would be foreign to it: every call S5_ERR_HIP)
        import torch  # noqa: F401
        L = ctypes.CDLL(lib_path)
        i64, vp, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.s5_discretize.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
        L.s5_discretize.restype = st
        L.s5_forward.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp]
        L.s5_forward.restype = st
        L.s5_forward_noalloc.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp]
        L.s5_forward_noalloc.restype = st
        L.s5_forward_timevarying.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp,
                                             vp, vp, vp, vp]
        L.s5_forward_timevarying.restype = st
        L.s5_forward_stateful.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp]
        L.s5_forward_stateful.restype = st
        L.s5_forward_timevarying_stateful.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp,
                                                      vp, vp, vp, vp, vp, vp, vp]
        L.s5_forward_timevarying_stateful.restype = st
        L.s5_forward_ex.argtypes = [ctypes.POINTER(ForwardDesc), vp]
        L.s5_forward_ex.restype = st
        L.s5_step.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_uint32] + [vp] * 10
        L.s5_step.restype = st
        L.s5_glu.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
        L.s5_glu.restype = st
        L.s5_status_string.argtypes = [st]
        L.s5_status_string.restype = ctypes.c_char_p
        L.s5_set_profiling_events.argtypes = [vp, ctypes.c_int]
        L.s5_set_profiling_events.restype = st
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().s5_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise S5Error(status, where)


def _stream_handle(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev_tensor(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return S5_F32
    if dtype == torch.bfloat16:
        return S5_BF16
    raise TypeError(f"u/y must be float32 or bfloat16, got {dtype}")


def discretize(lam, b_tilde, log_delta, lam_bar=None, b_bar=None, stream=None):
    """Zero-order hold: returns (Lambda_bar [P] complex64, B_bar [P,H] complex64)."""
    import torch
    P, H = b_tilde.shape
    _dev_tensor(lam, "lam", torch.complex64, (P,))
    _dev_tensor(b_tilde, "b_tilde", torch.complex64, (P, H))
    _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    if lam_bar is None:
        lam_bar = torch.empty(P, dtype=torch.complex64, device=lam.device)
    if b_bar is None:
        b_bar = torch.empty(P, H, dtype=torch.complex64, device=lam.device)
    _dev_tensor(lam_bar, "lam_bar", torch.complex64, (P,))
    _dev_tensor(b_bar, "b_bar", torch.complex64, (P, H))
    _check(lib().s5_discretize(P, H, lam.data_ptr(), b_tilde.data_ptr(), log_delta.data_ptr(),
                               lam_bar.data_ptr(), b_bar.data_ptr(), _stream_handle(stream)),
           "s5_discretize")
    return lam_bar, b_bar


def _forward_args(u, lam, b_tilde, c_tilde, d, y):
    import torch
    if u.dim() != 3:
        raise ValueError("u must be [B, L, H]")
    B, L, H = u.shape
    P = lam.shape[0]
    io = _io_code(u.dtype)
    _dev_tensor(u, "u", u.dtype, (B, L, H))
    _dev_tensor(lam, "lam", torch.complex64, (P,))
    _dev_tensor(b_tilde, "b_tilde", torch.complex64, (P, H))
    _dev_tensor(c_tilde, "c_tilde", torch.complex64, (H, P))
    _dev_tensor(d, "d", torch.float32, (H,))
    if y is None:
        y = torch.empty_like(u)
    _dev_tensor(y, "y", u.dtype, (B, L, H))
    return B, L, H, P, io, y


def forward(u, lam, b_tilde, c_tilde, d, log_delta, y=None, stream=None):
    """Time-invariant S5 forward: y = Re(C~ x_k) + D u_k, shape of u."""
    import torch
    B, L, H, P, io, y = _forward_args(u, lam, b_tilde, c_tilde, d, y)
    _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    _check(lib().s5_forward(B, L, H, P, io, u.data_ptr(), lam.data_ptr(), b_tilde.data_ptr(),
                            c_tilde.data_ptr(), d.data_ptr(), log_delta.data_ptr(), y.data_ptr(),
                            _stream_handle(stream)), "s5_forward")
    return y


def forward_noalloc(u, lam, b_tilde, c_tilde, d, log_delta, y=None, stream=None):
    """As forward, through s5_forward_noalloc: the library's scratch is its
    fixed per-device array (nothing is allocated by the library)."""
    import torch
    B, L, H, P, io, y = _forward_args(u, lam, b_tilde, c_tilde, d, y)
    _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    _check(lib().s5_forward_noalloc(B, L, H, P, io, u.data_ptr(), lam.data_ptr(), b_tilde.data_ptr(),
                                    c_tilde.data_ptr(), d.data_ptr(), log_delta.data_ptr(), y.data_ptr(),
                                    _stream_handle(stream)), "s5_forward_noalloc")
    return y


def forward_timevarying(u, lam, b_tilde, c_tilde, d, delta, y=None, stream=None):
    """S5 forward with one interval per (batch, step, mode): delta [B, L, P]."""
    import torch
    B, L, H, P, io, y = _forward_args(u, lam, b_tilde, c_tilde, d, y)
    _dev_tensor(delta, "delta", torch.float32, (B, L, P))
    _check(lib().s5_forward_timevarying(B, L, H, P, io, u.data_ptr(), lam.data_ptr(),
                                        b_tilde.data_ptr(), c_tilde.data_ptr(), d.data_ptr(),
                                        delta.data_ptr(), y.data_ptr(), _stream_handle(stream)),
           "s5_forward_timevarying")
    return y


def _state_args(x0, x_last, B, P, device):
    import torch
    if x0 is not None:
        _dev_tensor(x0, "x0", torch.complex64, (B, P))
    if x_last is None:
        x_last = torch.empty(B, P, dtype=torch.complex64, device=device)
    _dev_tensor(x_last, "x_last", torch.complex64, (B, P))
    return (x0.data_ptr() if x0 is not None else None), x_last


def forward_stateful(u, lam, b_tilde, c_tilde, d, log_delta, x0=None, y=None, x_last=None,
                     stream=None):
    """Time-invariant forward from the state x0 ([B, P] complex64, None = zero);
    returns (y, x_last) with x_last [B, P] the state after the last step."""
    import torch
    B, L, H, P, io, y = _forward_args(u, lam, b_tilde, c_tilde, d, y)
    _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    x0p, x_last = _state_args(x0, x_last, B, P, u.device)
    _check(lib().s5_forward_stateful(B, L, H, P, io, u.data_ptr(), lam.data_ptr(), b_tilde.data_ptr(),
                                     c_tilde.data_ptr(), d.data_ptr(), log_delta.data_ptr(), x0p,
                                     y.data_ptr(), x_last.data_ptr(), _stream_handle(stream)),
           "s5_forward_stateful")
    return y, x_last


def forward_timevarying_stateful(u, lam, b_tilde, c_tilde, d, delta, x0=None, y=None, x_last=None,
                                 stream=None):
    """Time-varying forward from the state x0; returns (y, x_last)."""
    import torch
    B, L, H, P, io, y = _forward_args(u, lam, b_tilde, c_tilde, d, y)
    _dev_tensor(delta, "delta", torch.float32, (B, L, P))
    x0p, x_last = _state_args(x0, x_last, B, P, u.device)
    _check(lib().s5_forward_timevarying_stateful(B, L, H, P, io, u.data_ptr(), lam.data_ptr(),
                                                 b_tilde.data_ptr(), c_tilde.data_ptr(), d.data_ptr(),
                                                 delta.data_ptr(), x0p, y.data_ptr(),
                                                 x_last.data_ptr(), _stream_handle(stream)),
           "s5_forward_timevarying_stateful")
    return y, x_last


def forward_ex(u, lam, b_tilde, c_tilde, d, log_delta=None, delta=None, x0=None, *,
               half_spectrum=False, bilinear=False, gelu=False, bidirectional=False,
               final_state=False, gelu_tanh=False, glu_w=None, glu_bias=None, glu_variant=1,
               y=None, x_last=None, stream=None):
    """The forward pass with its options (s5_forward_ex): exactly one of
    log_delta [P] (time-invariant) and delta [B, L, P] (time-varying);
    c_tilde [H, 2P] when bidirectional; glu_w [H, H] float32 (with glu_bias
    [H] or None, glu_variant 1 or 2) applies the gated activation to y.
    Returns (y, x_last), x_last None unless final_state is set or an x_last
    buffer is given."""
    import torch
    if u.dim() != 3:
        raise ValueError("u must be [B, L, H]")
    B, L, H = u.shape
    P = lam.shape[0]
    io = _io_code(u.dtype)
    _dev_tensor(u, "u", u.dtype, (B, L, H))
    _dev_tensor(lam, "lam", torch.complex64, (P,))
    _dev_tensor(b_tilde, "b_tilde", torch.complex64, (P, H))
    _dev_tensor(c_tilde, "c_tilde", torch.complex64, (H, 2 * P if bidirectional else P))
    _dev_tensor(d, "d", torch.float32, (H,))
    if (log_delta is None) == (delta is None):
        raise ValueError("give exactly one of log_delta and delta")
    if log_delta is not None:
        _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    if delta is not None:
        _dev_tensor(delta, "delta", torch.float32, (B, L, P))
    if y is None:
        y = torch.empty_like(u)
    _dev_tensor(y, "y", u.dtype, (B, L, H))
    x0p = None
    if x0 is not None:
        x0p = _dev_tensor(x0, "x0", torch.complex64, (B, P)).data_ptr()
    if final_state and x_last is None:
        x_last = torch.empty(B, P, dtype=torch.complex64, device=u.device)
    if x_last is not None:
        _dev_tensor(x_last, "x_last", torch.complex64, (B, P))
    if glu_w is not None:
        _dev_tensor(glu_w, "glu_w", torch.float32, (H, H))
        if glu_bias is not None:
            _dev_tensor(glu_bias, "glu_bias", torch.float32, (H,))
    flags = ((FLAG_HALF_SPECTRUM if half_spectrum else 0) | (FLAG_BILINEAR if bilinear else 0) |
             (FLAG_GELU if gelu else 0) | (FLAG_BIDIRECTIONAL if bidirectional else 0) |
             (FLAG_GELU_TANH if gelu_tanh else 0) | (FLAG_GLU if glu_w is not None else 0))
    desc = ForwardDesc(ctypes.sizeof(ForwardDesc), flags, io, B, L, H, P, u.data_ptr(), lam.data_ptr(),
                       b_tilde.data_ptr(), c_tilde.data_ptr(), d.data_ptr(),
                       log_delta.data_ptr() if log_delta is not None else None,
                       delta.data_ptr() if delta is not None else None, x0p, y.data_ptr(),
                       x_last.data_ptr() if x_last is not None else None,
                       glu_w.data_ptr() if glu_w is not None else None,
                       glu_bias.data_ptr() if glu_bias is not None and glu_w is not None else None,
                       glu_variant if glu_w is not None else 0)
    _check(lib().s5_forward_ex(ctypes.byref(desc), _stream_handle(stream)), "s5_forward_ex")
    return y, x_last


def step(u, lam, b_tilde, c_tilde, d, x, log_delta=None, delta=None, *, half_spectrum=False,
         bilinear=False, gelu=False, gelu_tanh=False, y=None, stream=None):
    """One recurrent step (s5_step): u [B, H]; x [B, P] complex64 updated in
    place; exactly one of log_delta [P] and delta [B, P]. Returns y [B, H]."""
    import torch
    if u.dim() != 2:
        raise ValueError("u must be [B, H]")
    B, H = u.shape
    P = lam.shape[0]
    io = _io_code(u.dtype)
    _dev_tensor(u, "u", u.dtype, (B, H))
    _dev_tensor(lam, "lam", torch.complex64, (P,))
    _dev_tensor(b_tilde, "b_tilde", torch.complex64, (P, H))
    _dev_tensor(c_tilde, "c_tilde", torch.complex64, (H, P))
    _dev_tensor(d, "d", torch.float32, (H,))
    _dev_tensor(x, "x", torch.complex64, (B, P))
    if (log_delta is None) == (delta is None):
        raise ValueError("give exactly one of log_delta and delta")
    if log_delta is not None:
        _dev_tensor(log_delta, "log_delta", torch.float32, (P,))
    if delta is not None:
        _dev_tensor(delta, "delta", torch.float32, (B, P))
    if y is None:
        y = torch.empty_like(u)
    _dev_tensor(y, "y", u.dtype, (B, H))
    flags = ((FLAG_HALF_SPECTRUM if half_spectrum else 0) | (FLAG_BILINEAR if bilinear else 0) |
             (FLAG_GELU if gelu else 0) | (FLAG_GELU_TANH if gelu_tanh else 0))
    _check(lib().s5_step(B, H, P, io, flags, u.data_ptr(), lam.data_ptr(), b_tilde.data_ptr(),
                         c_tilde.data_ptr(), d.data_ptr(),
                         log_delta.data_ptr() if log_delta is not None else None,
                         delta.data_ptr() if delta is not None else None, x.data_ptr(), y.data_ptr(),
                         _stream_handle(stream)), "s5_step")
    return y


def glu(y, w, bias=None, variant=1, out=None, stream=None):
    """Gated activation (s5_glu): y [..., H] float32 or bfloat16 (any leading
    shape, contiguous); w [H, H] float32; bias [H] float32 or None. Returns
    (variant 1) GELU(y) * sigmoid(GELU(y) w^T + b) or (variant 2)
    y * sigmoid(GELU(y) w^T + b); out may be y (in place)."""
    import torch
    H = y.shape[-1]
    T = y.numel() // H if H else 0
    io = _io_code(y.dtype)
    _dev_tensor(y, "y", y.dtype, tuple(y.shape))
    _dev_tensor(w, "w", torch.float32, (H, H))
    if bias is not None:
        _dev_tensor(bias, "bias", torch.float32, (H,))
    if out is None:
        out = torch.empty_like(y)
    _dev_tensor(out, "out", y.dtype, tuple(y.shape))
    _check(lib().s5_glu(T, H, io, int(variant), y.data_ptr(), w.data_ptr(),
                        bias.data_ptr() if bias is not None else None, out.data_ptr(),
                        _stream_handle(stream)), "s5_glu")
    return out


def set_profiling_events(events) -> None:
    """Raw hipEvent_t handles (ints), an even number up to 12: events[2k] and
    events[2k+1] are recorded around the k-th kernel launch (0 packing, 1
    aggregate pass, 2 state and output pass; 3-5 the same for the backward
    scan of the bidirectional form) of later forward calls from this thread.
    An empty sequence (or None) turns the hook off."""
    events = list(events or [])
    arr = (ctypes.c_void_p * max(1, len(events)))(*events) if events else None
    _check(lib().s5_set_profiling_events(arr, len(events)), "s5_set_profiling_events")
