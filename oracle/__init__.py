"""Tensor Cache CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference for the TC layer ("Tensor Cache:
Eviction-conditioned Associative Memory for Transformers", Sections 3.1-3.2,
Figure 2).  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it.  It shares no code with the HIP library
and never touches a GPU.

Contents
  * ``forward``, ``decode_step``, ``backward`` -- the per-token recurrence in
    IEEE double (``tc_oracle.c``), OpenMP over independent (b,h) pairs.
  * ``forward_chunk_mean`` -- the chunk-mean shortcut the exact scan
    replaces (one mean write per chunk of C evicted pairs), for the ablation.
  * ``forward_delta`` -- the optional delta-rule write (the evicted key's
    prediction error is written instead of its value), per token.
  * ``memory_f32_sequential`` / ``memory_f32_chunked`` -- float32 models of
    the memory path, per-token writes vs the chunked weighted-sum scan.
  * ``dense`` -- closed forms in numpy used to pin the oracle.

Every input is converted to float64 exactly (bf16 and fp32 values are exactly
representable), so the oracle reads the same numbers as the GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i = ctypes.c_int


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.tco_forward.argtypes = [_i] * 5 + [ctypes.c_double] + [_D] * 9
        lib.tco_decode_step.argtypes = [_i] * 4 + [ctypes.c_double] + [_D] * 6 + [_I64] + [_D] * 4
        lib.tco_backward.argtypes = [_i] * 5 + [ctypes.c_double] + [_D] * 13
        lib.tco_forward_chunk_mean.argtypes = [_i] * 6 + [ctypes.c_double] + [_D] * 9
        lib.tco_forward_delta.argtypes = [_i] * 5 + [ctypes.c_double] + [_D] * 9
        lib.tco_memory_f32_sequential.argtypes = [_i] * 3 + [ctypes.c_float] * 2 + [_F] * 5
        lib.tco_memory_f32_chunked.argtypes = [_i] * 4 + [ctypes.c_float] * 2 + [_F] * 5
        lib.tco_num_threads.restype = ctypes.c_int
        lib.tco_set_num_threads.argtypes = [_i]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().tco_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the following calls (timing only; results do not
    depend on it: the work is split per (b, h) and each is computed alone)."""
    _load().tco_set_num_threads(int(n))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: np.ndarray):
    return x.ctypes.data_as(_D)


def default_scale(D: int) -> float:
    """Softmax scale: the standard 1/sqrt(D) of scaled dot-product attention."""
    return 1.0 / np.sqrt(D)


def forward(q, k, v, lam, eta, gate, W: int, scale: float | None = None, with_state=True):
    """Per-token TC forward.  q,k,v: [B,H,T,D]; lam, eta, gate: [H].

    Returns (y [B,H,T,D], A_final [B,H,D,D], lse [B,H,T]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    lam, eta, gate = _f64(lam), _f64(eta), _f64(gate)
    assert lam.shape == eta.shape == gate.shape == (H,)
    tau = default_scale(D) if scale is None else float(scale)
    y = np.empty_like(q)
    A = np.empty((B, H, D, D))
    lse = np.empty((B, H, T))
    _load().tco_forward(B, H, T, D, int(W), tau, _p(q), _p(k), _p(v), _p(lam), _p(eta),
                        _p(gate), _p(y), _p(A), _p(lse))
    return y, A, lse


def forward_chunk_mean(q, k, v, lam, eta, gate, W: int, C: int, scale: float | None = None):
    """The chunk-mean shortcut's forward (what the exact scan replaces): one
    write A <- lam A + eta kbar vbar^T per chunk of C evicted pairs; a query
    whose evicted token lies in chunk n reads the memory after chunks
    0 .. n-1.  q,k,v: [B,H,T,D].  Returns (y, A_final after every complete
    chunk, lse) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    lam, eta, gate = _f64(lam), _f64(eta), _f64(gate)
    assert lam.shape == eta.shape == gate.shape == (H,) and int(C) >= 1
    tau = default_scale(D) if scale is None else float(scale)
    y = np.empty_like(q)
    A = np.empty((B, H, D, D))
    lse = np.empty((B, H, T))
    _load().tco_forward_chunk_mean(B, H, T, D, int(W), int(C), tau, _p(q), _p(k), _p(v), _p(lam), _p(eta),
                                   _p(gate), _p(y), _p(A), _p(lse))
    return y, A, lse


def forward_delta(q, k, v, lam, eta, gate, W: int, scale: float | None = None):
    """The delta-rule variant's forward (Figure 2, step 3, the optional
    write; reading: u = v_old - k_old A with A before the write, then
    A <- lam A + eta k_old u^T).  q,k,v: [B,H,T,D].  Returns (y, A_final,
    lse) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    lam, eta, gate = _f64(lam), _f64(eta), _f64(gate)
    assert lam.shape == eta.shape == gate.shape == (H,)
    tau = default_scale(D) if scale is None else float(scale)
    y = np.empty_like(q)
    A = np.empty((B, H, D, D))
    lse = np.empty((B, H, T))
    _load().tco_forward_delta(B, H, T, D, int(W), tau, _p(q), _p(k), _p(v), _p(lam), _p(eta), _p(gate), _p(y),
                              _p(A), _p(lse))
    return y, A, lse


def decode_step(q, k, v, k_ring, v_ring, A, pos, lam, eta, gate, scale: float | None = None):
    """One streaming step.  q,k,v: [S,H,D]; rings [S,H,W,D]; A [S,H,D,D];
    pos int64 [S].  Rings, A and pos are updated IN PLACE (float64 / int64
    arrays required); returns y [S,H,D]."""
    assert k_ring.dtype == np.float64 and v_ring.dtype == np.float64 and A.dtype == np.float64
    assert pos.dtype == np.int64 and k_ring.flags.c_contiguous and v_ring.flags.c_contiguous
    assert A.flags.c_contiguous and pos.flags.c_contiguous
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, H, D = q.shape
    W = k_ring.shape[2]
    lam, eta, gate = _f64(lam), _f64(eta), _f64(gate)
    tau = default_scale(D) if scale is None else float(scale)
    y = np.empty_like(q)
    _load().tco_decode_step(S, H, D, W, tau, _p(q), _p(k), _p(v), _p(k_ring), _p(v_ring),
                            _p(A), pos.ctypes.data_as(_I64), _p(lam), _p(eta), _p(gate), _p(y))
    return y


def forward_continue(q, k, v, k_ring, v_ring, A, pos0: int, lam, eta, gate,
                     scale: float | None = None):
    """T tokens of B sequences after ``pos0`` seen ones, by definition: T
    successive streaming steps (Figure 2), each one ``decode_step`` of the B
    sequences as streams.  q,k,v: [B,H,T,D]; rings [B,H,W,D] and A [B,H,D,D]
    (float64) are updated IN PLACE.  Returns y [B,H,T,D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    pos = np.full(B, int(pos0), np.int64)
    y = np.empty_like(q)
    for t in range(T):
        y[:, :, t] = decode_step(q[:, :, t], k[:, :, t], v[:, :, t], k_ring, v_ring, A, pos,
                                 lam, eta, gate, scale)
    return y


def backward(q, k, v, dy, lam, eta, gate, W: int, scale: float | None = None):
    """Gradients of L = sum <dy, y>.  Returns dq, dk, dv [B,H,T,D] and
    dlam, deta, dgate [H] (summed over the batch)."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, T, D = q.shape
    lam, eta, gate = _f64(lam), _f64(eta), _f64(gate)
    tau = default_scale(D) if scale is None else float(scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dl, de, dg = np.empty(H), np.empty(H), np.empty(H)
    _load().tco_backward(B, H, T, D, int(W), tau, _p(q), _p(k), _p(v), _p(dy), _p(lam),
                         _p(eta), _p(gate), _p(dq), _p(dk), _p(dv), _p(dl), _p(de), _p(dg))
    return dq, dk, dv, dl, de, dg


def _f32c(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def memory_f32_sequential(q, k, v, lam: float, eta: float, W: int):
    """float32 per-token writes; q,k,v [T,D].  Returns (m [T,D], A_final)."""
    q, k, v = _f32c(q), _f32c(k), _f32c(v)
    T, D = q.shape
    m = np.zeros((T, D), np.float32)
    A = np.zeros((D, D), np.float32)
    _load().tco_memory_f32_sequential(T, D, int(W), float(lam), float(eta), q.ctypes.data_as(_F),
                                      k.ctypes.data_as(_F), v.ctypes.data_as(_F),
                                      m.ctypes.data_as(_F), A.ctypes.data_as(_F))
    return m, A


def memory_f32_chunked(q, k, v, lam: float, eta: float, W: int, C: int):
    """float32 chunked weighted-sum scan; q,k,v [T,D].  Returns (m, A_final)."""
    q, k, v = _f32c(q), _f32c(k), _f32c(v)
    T, D = q.shape
    m = np.zeros((T, D), np.float32)
    A = np.zeros((D, D), np.float32)
    _load().tco_memory_f32_chunked(T, D, int(W), int(C), float(lam), float(eta),
                                   q.ctypes.data_as(_F), k.ctypes.data_as(_F),
                                   v.ctypes.data_as(_F), m.ctypes.data_as(_F),
                                   A.ctypes.data_as(_F))
    return m, A


from . import dense  # noqa: E402,F401
