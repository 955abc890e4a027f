"""Closed forms of the TC layer in numpy (float64) -- TEST INFRASTRUCTURE ONLY.

These restate what the per-token recurrence reaches in a different shape, so
that the C oracle can be pinned against them:

* ``closed_form_A``: unrolling the write A <- lambda*A + eta*k_w v_w^T of
  Section 3.2 / Figure 2 step 3 from A_0 = 0 gives
  A_t = sum_{i <= t-W} eta * lambda^(t-W-i) k_i v_i^T.
* ``dense_forward``: with the read identity q (k outer v) = <q,k> v of the
  abstract, the memory read is a masked, decayed linear attention, so the
  whole layer is one T x T computation:
  y = softmax_band(tau Q K^T) V + sigma(g) ((Q K^T) o L) V,
  L[t,i] = eta * lambda^(t-W-i) for i <= t-W, 0 otherwise.
* ``chunk_mean_write``: the chunk-mean shortcut of the abstract,
  A <- lambda*A + eta*(kbar outer vbar), used only to check the pages'
  C^2 - C cross-term statement.
* ``state_after_writes``: A after writing a list of pairs in order; used to
  build decode start states from prior evictions.
"""
from __future__ import annotations

import numpy as np


def closed_form_A(k: np.ndarray, v: np.ndarray, lam: float, eta: float, W: int, t: int):
    """A_t for one head; k, v [T, D]; returns D x D (zero while t < W)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    D = k.shape[1]
    A = np.zeros((D, D))
    for i in range(0, t - W + 1):
        A += eta * lam ** (t - W - i) * np.outer(k[i], v[i])
    return A


def memory_weights(T: int, W: int, lam: float, eta: float) -> np.ndarray:
    """L[t, i] = eta*lambda^(t-W-i) if i <= t-W else 0  (T x T)."""
    t = np.arange(T)[:, None]
    i = np.arange(T)[None, :]
    lag = t - W - i
    L = np.where(lag >= 0, eta * np.power(float(lam), np.maximum(lag, 0)), 0.0)
    return L


def band_mask(T: int, W: int) -> np.ndarray:
    """True where key i is in the window of query t: t-W < i <= t."""
    t = np.arange(T)[:, None]
    i = np.arange(T)[None, :]
    return (i <= t) & (i > t - W)


def dense_forward(q, k, v, lam, eta, gate, W: int, scale: float):
    """Single head O(T^2) form; q, k, v [T, D].  Returns y [T, D], lse [T]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T = q.shape[0]
    Z = q @ k.T
    S = np.where(band_mask(T, W), scale * Z, -np.inf)
    mu = S.max(axis=1, keepdims=True)
    E = np.exp(S - mu)
    ell = E.sum(axis=1, keepdims=True)
    y_local = (E / ell) @ v
    sg = 1.0 / (1.0 + np.exp(-float(gate)))
    m = (Z * memory_weights(T, W, lam, eta)) @ v
    return y_local + sg * m, (mu + np.log(ell))[:, 0]


def chunk_mean_write(A, k_chunk, v_chunk, lam: float, eta: float):
    """The chunk-mean shortcut: A <- lam*A + eta * kbar vbar^T for one chunk."""
    kb = np.asarray(k_chunk, np.float64).mean(axis=0)
    vb = np.asarray(v_chunk, np.float64).mean(axis=0)
    return lam * np.asarray(A, np.float64) + eta * np.outer(kb, vb)


def state_after_writes(k, v, lam: float, eta: float):
    """A after writing rows 0..n-1 of k, v (each [..., n, D]) in order from
    A = 0:  sum_i eta*lam^(n-1-i) k_i v_i^T.  float64; leading dims batched."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = k.shape[-2]
    lam = np.asarray(lam, np.float64)
    eta = np.asarray(eta, np.float64)
    # weights [..., n]; lam/eta broadcast over the leading dims
    expo = np.arange(n - 1, -1, -1, dtype=np.float64)
    w = eta[..., None] * np.power(lam[..., None], expo)
    return np.matmul(np.swapaxes(k, -1, -2), w[..., :, None] * v)
