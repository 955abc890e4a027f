"""Python binding of the TC C ABI (include/tc.h) -- argument marshalling only.

Every step of the layer runs in the HIP kernels of ``libtc.so``; this module
only checks tensor metadata against the documented layouts (shape, dtype,
device, contiguity: the library receives bare pointers and cannot check
sizes), allocates outputs/workspaces with torch (device memory plumbing) and
passes raw device pointers plus the current HIP stream.
If the library has not been built it raises; there is no fallback.

Entry points mirror the C names: ``tc_forward``, ``tc_decode_step``,
``tc_forward_continue``, ``tc_backward``, ``tc_forward_workspace_size``,
``tc_continue_workspace_size``, ``tc_backward_workspace_size``,
``tc_forward_status``, ``tc_forward_noalloc``, ``tc_forward_chunk_mean``, ``tc_forward_delta``,
``tc_status_string``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtc.so")

TC_OK, TC_ERR_INVALID_ARGUMENT, TC_ERR_UNSUPPORTED, TC_ERR_WORKSPACE, TC_ERR_HIP, TC_ERR_STATE_EXCHANGE = range(6)
TC_F32, TC_BF16 = 0, 1


class TCError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, tc_status_string(status), status))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("D", ctypes.c_int32), ("W", ctypes.c_int32), ("C", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class DecodeShape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("W", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libtc.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtc.so is not built (run: python -m eviction_fed_weight_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.tc_forward_workspace_size.argtypes = [ctypes.POINTER(Shape)]
        L.tc_forward_workspace_size.restype = _sz
        L.tc_backward_workspace_size.argtypes = [ctypes.POINTER(Shape)]
        L.tc_backward_workspace_size.restype = _sz
        L.tc_forward.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 10 + [_sz, _vp]
        L.tc_forward.restype = ctypes.c_int
        L.tc_decode_step.argtypes = [ctypes.POINTER(DecodeShape)] + [_vp] * 12
        L.tc_decode_step.restype = ctypes.c_int
        L.tc_continue_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64]
        L.tc_continue_workspace_size.restype = _sz
        L.tc_forward_continue.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64] + [_vp] * 13 + [_sz, _vp]
        L.tc_forward_continue.restype = ctypes.c_int
        L.tc_forward_chunk_mean.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 10 + [_sz, _vp]
        L.tc_forward_chunk_mean.restype = ctypes.c_int
        L.tc_forward_delta_workspace_size.argtypes = [ctypes.POINTER(Shape)]
        L.tc_forward_delta_workspace_size.restype = _sz
        L.tc_forward_delta.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 10 + [_sz, _vp]
        L.tc_forward_delta.restype = ctypes.c_int
        L.tc_forward_noalloc.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 10
        L.tc_forward_noalloc.restype = ctypes.c_int
        L.tc_forward_status.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64, _vp, _sz, _vp]
        L.tc_forward_status.restype = ctypes.c_int
        L.tc_backward.argtypes = [ctypes.POINTER(Shape)] + [_vp] * 16 + [_sz, _vp]
        L.tc_backward.restype = ctypes.c_int
        L.tc_status_string.argtypes = [ctypes.c_int]
        L.tc_status_string.restype = ctypes.c_char_p
        L.tc_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def tc_status_string(status: int) -> str:
    return lib().tc_status_string(int(status)).decode()


def tc_version() -> str:
    return lib().tc_version().decode()


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TC_BF16
    if t.dtype == torch.float32:
        return TC_F32
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _want(t, name, shape, dtype, device=None):
    """Check one tensor argument against the layout the C ABI documents for
    it (the library receives bare pointers and cannot check sizes itself):
    exact shape, element type, contiguity and, once the first tensor's
    device is known, the same device.  Raises ValueError naming the tensor."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s: on %s, expected %s (the device of q)" % (name, t.device, device))


def _want_params(H, dev, **params):
    """lambda, eta, gate: float32 vectors of H elements."""
    torch = _torch()
    for name, t in params.items():
        if t is None:
            raise ValueError("%s is required" % name)
        _want(t, name, (H,), torch.float32, dev)


def _stream(device=None):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def make_shape(B, H, T, D, W, C=64, scale=0.0, dtype=TC_BF16) -> Shape:
    return Shape(int(B), int(H), int(T), int(D), int(W), int(C), float(scale), int(dtype))


def tc_forward_workspace_size(shape: Shape) -> int:
    return int(lib().tc_forward_workspace_size(ctypes.byref(shape)))


def tc_backward_workspace_size(shape: Shape) -> int:
    return int(lib().tc_backward_workspace_size(ctypes.byref(shape)))


def _workspace(nbytes, device, ws):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("ws: must be a contiguous tensor on %s" % device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small: %d < %d bytes" % (ws.numel() * ws.element_size(), nbytes))
    return ws, ws.numel() * ws.element_size()


def tc_forward(q, k, v, lam, eta, gate, W: int, C: int = 64, scale: float = 0.0, *,
               want_state: bool = True, want_lse: bool = True, y=None, A_final=None, lse=None,
               ws=None):
    """Prefill/training forward.  q, k, v: [B,H,T,D] (bf16 or fp32, CUDA);
    lam, eta, gate: [H] float32.  Returns (y, A_final or None, lse or None)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    B, H, T, D = q.shape
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    _want(A_final, "A_final", (B, H, D, D), torch.float32, dev)
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    if y is None:
        y = torch.empty_like(q)
    if want_state and A_final is None:
        A_final = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(tc_forward_workspace_size(shape), dev, ws)
    st = lib().tc_forward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(eta),
                          _ptr(gate), _ptr(y), _ptr(A_final) if want_state else None,
                          _ptr(lse) if want_lse else None, _ptr(ws) if ws is not None else None,
                          wsb, _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_forward")
    return y, (A_final if want_state else None), (lse if want_lse else None)


def tc_forward_delta_workspace_size(shape) -> int:
    return int(lib().tc_forward_delta_workspace_size(ctypes.byref(shape)))


def tc_forward_delta(q, k, v, lam, eta, gate, W: int, C: int = 64, scale: float = 0.0, *,
                     want_state: bool = True, want_lse: bool = True, y=None, A_final=None, lse=None, ws=None):
    """The layer with the delta-rule write (the evicted key's prediction
    error is written).  Arguments and returns as tc_forward; its own workspace
    (tc_forward_delta_workspace_size)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    B, H, T, D = q.shape
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    _want(A_final, "A_final", (B, H, D, D), torch.float32, dev)
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    if y is None:
        y = torch.empty_like(q)
    if want_state and A_final is None:
        A_final = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(tc_forward_delta_workspace_size(shape), dev, ws)
    st = lib().tc_forward_delta(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(eta), _ptr(gate),
                                _ptr(y), _ptr(A_final) if want_state else None, _ptr(lse) if want_lse else None,
                                _ptr(ws) if ws is not None else None, wsb, _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_forward_delta")
    return y, (A_final if want_state else None), (lse if want_lse else None)


def tc_forward_chunk_mean(q, k, v, lam, eta, gate, W: int, C: int, scale: float = 0.0, *,
                          want_state: bool = True, want_lse: bool = True, y=None, A_final=None, lse=None, ws=None):
    """The chunk-mean shortcut's forward (one mean write per chunk of C
    evicted pairs; the ablation of the exact scan).  Arguments and returns as
    tc_forward; bf16, D <= 64, C in {64, 128}, W a multiple of C."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    B, H, T, D = q.shape
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    _want(A_final, "A_final", (B, H, D, D), torch.float32, dev)
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    if y is None:
        y = torch.empty_like(q)
    if want_state and A_final is None:
        A_final = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(tc_forward_workspace_size(shape), dev, ws)
    st = lib().tc_forward_chunk_mean(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(eta),
                                     _ptr(gate), _ptr(y), _ptr(A_final) if want_state else None,
                                     _ptr(lse) if want_lse else None, _ptr(ws) if ws is not None else None,
                                     wsb, _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_forward_chunk_mean")
    return y, (A_final if want_state else None), (lse if want_lse else None)


NOALLOC_SCRATCH_BYTES = 32 << 20  # the static device scratch of tc_forward_noalloc


def tc_forward_noalloc(q, k, v, lam, eta, gate, W: int, C: int = 64, scale: float = 0.0, *, y, A_final=None,
                       lse=None):
    """tc_forward without a workspace: the library uses its static 32 MiB
    device scratch (no device allocation in the call).  The outputs are
    passed in (y required; A_final and lse optional).  Returns (y, A_final,
    lse)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    if y is None:
        raise ValueError("y is required")
    B, H, T, D = q.shape
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    _want(A_final, "A_final", (B, H, D, D), torch.float32, dev)
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    st = lib().tc_forward_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(eta),
                                  _ptr(gate), _ptr(y), _ptr(A_final), _ptr(lse), _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_forward_noalloc")
    return y, A_final, lse


def tc_decode_step(q, k, v, k_ring, v_ring, A, pos, lam, eta, gate, scale: float = 0.0, *, y=None):
    """One decode step for S streams.  q, k, v: [S,H,D]; rings [S,H,W,D]
    (updated in place); A [S,H,D,D] float32 (in place); pos [S] int64 (+1).
    Returns y [S,H,D]."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q: expected [S,H,D], got shape %s" % (tuple(q.shape),))
    if k_ring.dim() != 4:
        raise ValueError("k_ring: expected [S,H,W,D], got shape %s" % (tuple(k_ring.shape),))
    S, H, D = q.shape
    W = k_ring.shape[2]
    shape = DecodeShape(S, H, D, W, float(scale), _dtype_code(q))
    dv = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dv)
    _want(k_ring, "k_ring", (S, H, W, D), q.dtype, dv)
    _want(v_ring, "v_ring", (S, H, W, D), q.dtype, dv)
    _want(A, "A", (S, H, D, D), torch.float32, dv)
    _want(pos, "pos", (S,), torch.int64, dv)
    _want_params(H, dv, lam=lam, eta=eta, gate=gate)
    if y is None:
        y = torch.empty_like(q)
    st = lib().tc_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_ring),
                              _ptr(v_ring), _ptr(A), _ptr(pos), _ptr(lam), _ptr(eta), _ptr(gate),
                              _ptr(y), _stream(q.device))
    if st != TC_OK:
        raise TCError(st, "tc_decode_step")
    return y


def tc_continue_workspace_size(shape: Shape, pos0: int) -> int:
    return int(lib().tc_continue_workspace_size(ctypes.byref(shape), int(pos0)))


def tc_forward_continue(q, k, v, lam, eta, gate, k_ring, v_ring, A, pos0: int, *, pos=None, C: int = 64,
                        scale: float = 0.0, want_lse: bool = True, y=None, lse=None, ws=None):
    """The next T tokens of B sequences that have seen ``pos0`` tokens.
    q, k, v: [B,H,T,D]; rings [B,H,W,D] and A [B,H,D,D] float32 are updated
    in place (the decode layout with S = B); pos ([B] int64, optional) is set
    to pos0 + T.  Returns (y, lse or None)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    if k_ring.dim() != 4:
        raise ValueError("k_ring: expected [B,H,W,D], got shape %s" % (tuple(k_ring.shape),))
    B, H, T, D = q.shape
    W = k_ring.shape[2]
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y)):
        _want(t, name, q.shape, q.dtype, dev)
    _want(k_ring, "k_ring", (B, H, W, D), q.dtype, dev)
    _want(v_ring, "v_ring", (B, H, W, D), q.dtype, dev)
    _want(A, "A", (B, H, D, D), torch.float32, dev)
    _want(pos, "pos", (B,), torch.int64, dev)
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    if y is None:
        y = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(tc_continue_workspace_size(shape, pos0), dev, ws)
    st = lib().tc_forward_continue(ctypes.byref(shape), int(pos0), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                   _ptr(eta), _ptr(gate), _ptr(k_ring), _ptr(v_ring), _ptr(A),
                                   _ptr(pos) if pos is not None else None, _ptr(y),
                                   _ptr(lse) if want_lse else None, _ptr(ws) if ws is not None else None,
                                   wsb, _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_forward_continue")
    return y, (lse if want_lse else None)


def tc_forward_status(shape: Shape, ws, pos0: int = 0) -> int:
    """Status of the last forward call (tc_forward: pos0 = 0, or
    tc_forward_continue with its pos0) that used workspace ``ws`` (a torch
    tensor or None): TC_OK, or TC_ERR_STATE_EXCHANGE when one of its flag
    waits ran out.  Synchronises the current stream."""
    p = _ptr(ws) if ws is not None else None
    n = ws.numel() * ws.element_size() if ws is not None else 0
    dev = ws.device if ws is not None else None
    return int(lib().tc_forward_status(ctypes.byref(shape), int(pos0), p, n, _stream(dev)))


def tc_backward(q, k, v, y, dy, lse, lam, eta, gate, W: int, C: int = 64, scale: float = 0.0, *,
                dq=None, dk=None, dv=None, ws=None):
    """Gradients of sum <dy, y>.  Returns dq, dk, dv, dlam, deta, dgate."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q: expected [B,H,T,D], got shape %s" % (tuple(q.shape),))
    B, H, T, D = q.shape
    shape = make_shape(B, H, T, D, W, C, scale, _dtype_code(q))
    dev = q.device
    for name, t in (("k", k), ("v", v), ("y", y), ("dy", dy), ("dq", dq), ("dk", dk), ("dv", dv)):
        _want(t, name, q.shape, q.dtype, dev)
    if y is None or dy is None or lse is None:
        raise ValueError("y, dy and lse are required")
    _want(lse, "lse", (B, H, T), torch.float32, dev)
    _want_params(H, dev, lam=lam, eta=eta, gate=gate)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    dl = torch.empty(H, dtype=torch.float32, device=dev)
    de = torch.empty(H, dtype=torch.float32, device=dev)
    dg = torch.empty(H, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(tc_backward_workspace_size(shape), dev, ws)
    st = lib().tc_backward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy),
                           _ptr(lse), _ptr(lam), _ptr(eta), _ptr(gate), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(dl), _ptr(de), _ptr(dg), _ptr(ws) if ws is not None else None, wsb,
                           _stream(dev))
    if st != TC_OK:
        raise TCError(st, "tc_backward")
    return dq, dk, dv, dl, de, dg
