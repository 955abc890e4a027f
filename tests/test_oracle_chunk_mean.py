"""Pins of the chunk-mean shortcut in the oracle (oracle.forward_chunk_mean),
the write A <- lam A + eta (kbar outer vbar) per chunk of C evicted pairs
that the abstract, Section 1 (contributions) and Section 2 of "Tensor Cache:
Eviction-conditioned Associative Memory for Transformers" name as what the
exact scan replaces.  Reading pinned here: a query whose evicted token lies
in chunk n reads the memory after chunks 0 .. n-1; A_final holds every
complete chunk.  Each pin comes from outside the oracle's own loop: a
brute-force closed form over the chunk means, the exact layer at window
W + 1 (C = 1), a lone chunk, the pages' C^2 - C cross terms (lam = 1), and
the pure sliding window (T <= W)."""
import numpy as np
import pytest

import oracle
from oracle import dense


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def local_only(q, k, v, W):
    """y_local (the window softmax alone): the exact oracle with eta = 0."""
    H = q.shape[1]
    y, _, _ = oracle.forward(q, k, v, np.full(H, 0.5), np.zeros(H), np.zeros(H), W)
    return y


@pytest.mark.parametrize("T,W,C,lam", [(20, 4, 3, 0.8), (23, 5, 4, 0.9), (17, 2, 5, 1.0), (30, 6, 3, 0.0)])
def test_closed_form_over_chunk_means(T, W, C, lam):
    """Every row's memory read and A_final against the sum over chunk means
    written out by brute force (incomplete last chunk left out of A_final)."""
    D, eta, g = 3, 0.7, 0.4
    q, k, v = (rnd((1, 1, T, D), s) for s in (1, 2, 3))
    y, A, _ = oracle.forward_chunk_mean(q, k, v, np.array([lam]), np.array([eta]), np.array([g]), W, C)
    sig = 1 / (1 + np.exp(-g))
    m = (y - local_only(q, k, v, W))[0, 0] / sig
    E = max(T - W, 0)
    means = [(k[0, 0, n * C:(n + 1) * C].mean(0), v[0, 0, n * C:(n + 1) * C].mean(0)) for n in range(E // C)]

    def state(nchunks):
        S = np.zeros((D, D))
        for i in range(nchunks):
            S += eta * lam ** (nchunks - 1 - i) * np.outer(*means[i])
        return S

    for t in range(T):
        expect = np.zeros(D) if t < W else q[0, 0, t] @ state((t - W) // C)
        assert np.allclose(m[t], expect, atol=1e-12), t
    assert np.allclose(A[0, 0], state(E // C), atol=1e-12)


def test_chunk_of_one_is_the_exact_memory_one_step_late():
    """C = 1: chunk n is the single token n, read only from step n + W + 1 on,
    so the memory read equals the exact layer's with window W + 1 (dense
    masked form), while L1 keeps window W."""
    B, H, T, D, W = 1, 2, 40, 4, 6
    q, k, v = (rnd((B, H, T, D), s) for s in (4, 5, 6))
    lam, eta, g = np.array([0.9, 0.6]), np.array([0.5, 1.5]), np.array([0.3, -1.0])
    y, A, _ = oracle.forward_chunk_mean(q, k, v, lam, eta, g, W, 1)
    yl = local_only(q, k, v, W)
    for h in range(H):
        Z = q[0, h] @ k[0, h].T
        m = (Z * dense.memory_weights(T, W + 1, lam[h], eta[h])) @ v[0, h]
        sig = 1 / (1 + np.exp(-g[h]))
        assert np.allclose(y[0, h], yl[0, h] + sig * m, atol=1e-12)
        # all T - W tokens written: the exact closed form at the last step
        assert np.allclose(A[0, h], dense.closed_form_A(k[0, h], v[0, h], lam[h], eta[h], W, T - 1), atol=1e-12)


def test_one_chunk_is_read_by_nobody():
    """C = T - W: the only chunk completes at the last step, so every read is
    zero (y = y_local) and A_final = eta kbar vbar^T."""
    T, D, W = 25, 4, 5
    q, k, v = (rnd((1, 1, T, D), s) for s in (7, 8, 9))
    y, A, _ = oracle.forward_chunk_mean(q, k, v, np.array([0.7]), np.array([0.9]), np.array([2.0]), W, T - W)
    assert np.allclose(y, local_only(q, k, v, W), atol=1e-13)
    assert np.allclose(A[0, 0], 0.9 * np.outer(k[0, 0, :T - W].mean(0), v[0, 0, :T - W].mean(0)), atol=1e-13)


@pytest.mark.parametrize("C", [2, 4, 7])
def test_c2_minus_c_cross_terms_against_the_exact_memory(C):
    """lam = 1: C^2 times the shortcut's memory minus the exact memory of the
    same evictions is the sum of the C^2 - C cross products k_i v_j^T (i != j,
    both in one chunk) of every chunk, enumerated one by one."""
    nch, D, W, eta = 3, 3, 4, 0.6
    T = W + nch * C
    q, k, v = (rnd((1, 1, T, D), s) for s in (10, 11, 12))
    one = np.array([1.0])
    _, A_sc, _ = oracle.forward_chunk_mean(q, k, v, one, np.array([eta]), np.zeros(1), W, C)
    _, A_ex, _ = oracle.forward(q, k, v, one, np.array([eta]), np.zeros(1), W)
    cross, count = np.zeros((D, D)), 0
    for n in range(nch):
        for i in range(n * C, (n + 1) * C):
            for j in range(n * C, (n + 1) * C):
                if i != j:
                    cross += eta * np.outer(k[0, 0, i], v[0, 0, j])
                    count += 1
    assert count == nch * (C * C - C)
    assert np.allclose(C * C * A_sc[0, 0] - A_ex[0, 0], cross, atol=1e-12)


def test_no_eviction_is_the_sliding_window():
    T, D, W = 12, 4, 12
    q, k, v = (rnd((1, 1, T, D), s) for s in (13, 14, 15))
    y, A, _ = oracle.forward_chunk_mean(q, k, v, np.array([0.9]), np.array([0.5]), np.array([1.0]), W, 4)
    assert np.allclose(y, local_only(q, k, v, W), atol=1e-13) and not A.any()
