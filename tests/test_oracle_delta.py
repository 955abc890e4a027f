"""Pins of the oracle's delta-rule forward (the optional write of Figure 2,
step 3, in the Widrow-Hoff error-correcting reading: u = v_old - k_old A with
A before the write, then A <- lambda A + eta k_old u^T).

Each pin is fixed by the mathematics, not by the oracle's code: a reduction
to the outer-product write when every prediction vanishes, hand-derived
closed forms of two writes of one key, the exact-recall property of an
error-correcting write with unit keys, and the trivial limits.
"""
import numpy as np
import pytest

import oracle


def _params(H, lam, eta, gate=0.0):
    return np.full(H, lam), np.full(H, eta), np.full(H, gate)


def test_delta_equals_outer_product_when_predictions_vanish():
    # orthonormal keys, each evicted once: every prediction k_e A is zero, so
    # the delta write is the outer-product write and the layers agree
    rng = np.random.default_rng(1)
    B, H, D, W = 1, 2, 8, 3
    T = W + D
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = rng.standard_normal((B, H, T, D)) * 0.3
    for h in range(H):
        k[0, h, :D] = np.roll(Qm, h, axis=0)  # tokens 0 .. D-1 are the evicted ones
    q = rng.standard_normal((B, H, T, D))
    v = rng.standard_normal((B, H, T, D))
    lam, eta, g = np.array([0.9, 0.7]), np.array([0.5, 1.3]), np.array([0.3, -1.0])
    y1, A1, l1 = oracle.forward_delta(q, k, v, lam, eta, g, W)
    y0, A0, l0 = oracle.forward(q, k, v, lam, eta, g, W)
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(A1, A0, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(l1, l0)


@pytest.mark.parametrize("lam,eta", [(1.0, 1.0), (0.8, 0.3), (0.95, 1.7)])
def test_two_writes_of_one_key_closed_form(lam, eta):
    # W = 1, tokens (e1, a), (e1, b), (e2, c): two evictions of key e1.
    # First write: A1 = eta e1 a^T.  Prediction of the second: e1 A1 = eta a,
    # so A2 = lam eta e1 a^T + eta e1 (b - eta a)^T
    #       = e1 (eta (lam - eta) a + eta b)^T.
    D = 4
    a = np.array([1.0, -2.0, 0.5, 3.0])
    b = np.array([0.25, 1.0, -1.0, 2.0])
    c = np.array([7.0, 0.0, 1.0, -1.0])
    e1, e2 = np.eye(D)[0], np.eye(D)[1]
    k = np.stack([e1, e1, e2])[None, None]
    v = np.stack([a, b, c])[None, None]
    q = np.zeros_like(k)
    _, A, _ = oracle.forward_delta(q, k, v, *_params(1, lam, eta), 1)
    want = np.outer(e1, eta * (lam - eta) * a + eta * b)
    np.testing.assert_allclose(A[0, 0], want, rtol=0, atol=1e-14)
    # with lam = eta = 1 the second write replaces the first value
    if lam == 1.0 and eta == 1.0:
        np.testing.assert_allclose(A[0, 0], np.outer(e1, b), rtol=0, atol=1e-15)


def test_unit_key_write_recalls_exactly():
    # lam = eta = 1 and |k| = 1: after writing (k, v) the memory returns v for
    # k, whatever it held before (k A' = k A + |k|^2 (v - k A) = v)
    rng = np.random.default_rng(2)
    D, W, T = 6, 2, 14
    k = rng.standard_normal((1, 1, T, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, D))
    q = rng.standard_normal((1, 1, T, D))
    for Tp in range(W + 1, T + 1):
        _, A, _ = oracle.forward_delta(q[:, :, :Tp], k[:, :, :Tp], v[:, :, :Tp], *_params(1, 1.0, 1.0), W)
        e = Tp - 1 - W  # the last evicted token
        np.testing.assert_allclose(k[0, 0, e] @ A[0, 0], v[0, 0, e], rtol=0, atol=1e-12)


def test_decay_only_off_the_written_key():
    # one write changes A only along the written key: for x orthogonal to k_e,
    # x A_{e+1} = lam x A_e
    rng = np.random.default_rng(3)
    D, W, T = 5, 2, 9
    k = rng.standard_normal((1, 1, T, D)) / np.sqrt(D)
    v = rng.standard_normal((1, 1, T, D))
    q = np.zeros((1, 1, T, D))
    lam, eta = 0.85, 0.6
    _, A0, _ = oracle.forward_delta(q[:, :, :T - 1], k[:, :, :T - 1], v[:, :, :T - 1], *_params(1, lam, eta), W)
    _, A1, _ = oracle.forward_delta(q, k, v, *_params(1, lam, eta), W)
    ke = k[0, 0, T - 1 - W]
    x = rng.standard_normal(D)
    x -= (x @ ke) / (ke @ ke) * ke
    np.testing.assert_allclose(x @ A1[0, 0], lam * (x @ A0[0, 0]), rtol=0, atol=1e-12)
    # and along k_e: k A_{e+1} = (lam - eta |k|^2) k A_e + eta |k|^2 v_e
    n2 = ke @ ke
    np.testing.assert_allclose(ke @ A1[0, 0], (lam - eta * n2) * (ke @ A0[0, 0]) + eta * n2 * v[0, 0, T - 1 - W],
                               rtol=0, atol=1e-12)


def test_delta_limits():
    rng = np.random.default_rng(4)
    B, H, T, D = 1, 2, 30, 8
    q, k, v = (rng.standard_normal((B, H, T, D)) / np.sqrt(D) for _ in range(3))
    # no eviction (W >= T): the same layer as the outer-product write
    y1, A1, _ = oracle.forward_delta(q, k, v, *_params(H, 0.9, 0.5), T)
    y0, _, _ = oracle.forward(q, k, v, *_params(H, 0.9, 0.5), T)
    np.testing.assert_array_equal(y1, y0)
    assert not A1.any()
    # eta = 0: nothing is written
    y1, A1, _ = oracle.forward_delta(q, k, v, *_params(H, 0.9, 0.0), 4)
    y0, _, _ = oracle.forward(q, k, v, *_params(H, 0.9, 0.0), 4)
    np.testing.assert_array_equal(y1, y0)
    assert not A1.any()
