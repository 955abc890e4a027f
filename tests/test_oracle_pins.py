"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the per-token recurrence (oracle/tc_oracle.c) against
something other than itself: a closed form, a hand-worked example, a library
routine the layer reduces to in a special case, or an invariant stated on the
pages ("Tensor Cache: Eviction-conditioned Associative Memory for
Transformers": Section 3.1 Eq. (1) window attention; Section 3.2 / Figure 2
eviction-conditioned write, read and gate; abstract: read identity,
chunk-mean shortcut and the parallel weighted-sum scan).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import dense

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def one_head(T, D, seed=0):
    q, k, v = rnd(seed, T, D), rnd(seed + 1, T, D), rnd(seed + 2, T, D)
    return q, k, v


def fwd1(q, k, v, lam, eta, g, W, scale=None):
    y, A, lse = oracle.forward(q[None, None], k[None, None], v[None, None], [lam], [eta], [g], W, scale)
    return y[0, 0], A[0, 0], lse[0, 0]


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


# --------------------------------------------------------------------------- state


@pytest.mark.parametrize("T,D,W,lam,eta", [(20, 4, 3, 0.7, 0.4), (33, 5, 1, 0.95, 1.3), (17, 3, 16, 0.5, 0.2),
                                           (12, 2, 12, 0.9, 0.9), (25, 6, 7, 0.0, 0.5), (25, 6, 7, 1.0, 0.5)])
def test_state_matches_closed_form(T, D, W, lam, eta):
    """Unrolled write: A_t = sum_{i<=t-W} eta lam^(t-W-i) k_i v_i^T, for every t."""
    q, k, v = one_head(T, D, 3)
    for t in range(T):
        _, A, _ = fwd1(q[: t + 1], k[: t + 1], v[: t + 1], lam, eta, 0.3, W)
        np.testing.assert_allclose(A, dense.closed_form_A(k, v, lam, eta, W, t), rtol=1e-12, atol=1e-12)


def test_state_is_k_outer_v_not_v_outer_k():
    """k outer v = k v^T: A[a][c] = eta k[a] v[c] after one eviction."""
    k = np.array([[2.0, 1.0], [0.0, 0.0]])
    v = np.array([[0.0, 3.0], [0.0, 0.0]])
    q = np.array([[1.0, 0.0], [1.0, 0.0]])
    _, A, _ = fwd1(q, k, v, 0.5, 0.25, 0.0, 1)
    np.testing.assert_array_equal(A, 0.25 * np.array([[0.0, 6.0], [0.0, 3.0]]))


# --------------------------------------------------------------------------- hand examples


def test_hand_example_d1():
    """D=1, W=1, tau=1, lam=1/2, eta=1/4, g=0 (sigma=1/2).  By hand:
    window = {t} so y_local = v_t and lse_t = q_t k_t;  A_0 = 0,
    A_1 = eta k0 v0 = 1/4,  A_2 = lam A_1 + eta k1 v1 = 1/8 - 3/4 = -5/8;
    y = [2, 3 + 1/2*2*1/4, -1 + 1/2*3*(-5/8)] = [2, 13/4, -31/16]."""
    q = np.array([[1.0], [2.0], [3.0]])
    k = np.array([[0.5], [-1.0], [2.0]])
    v = np.array([[2.0], [3.0], [-1.0]])
    y, A, lse = fwd1(q, k, v, 0.5, 0.25, 0.0, 1, scale=1.0)
    np.testing.assert_allclose(y[:, 0], [2.0, 13.0 / 4.0, -31.0 / 16.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(A, [[-5.0 / 8.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, [0.5, -2.0, 6.0], rtol=0, atol=1e-15)


def test_hand_example_window2():
    """D=2, W=2, tau=1, lam=1, eta=1, g=ln(3) (sigma=3/4), T=3.
    q_t = (1,0) for all t; k = [(0,0),(ln2,0),(0,5)]; v = [(1,0),(0,1),(2,2)].
    t=0: window {0}: y_local = v0 = (1,0), lse = 0.
    t=1: window {0,1}, scores (0, ln2) -> weights (1/3, 2/3):
         y_local = (1/3, 2/3), lse = ln 3.
    t=2: token 0 evicted, A_2 = k0 v0^T = 0 -> m = 0;
         window {1,2}, scores (ln2, 0) -> weights (2/3, 1/3):
         y_local = (2/3, 2/3 + ... ) = (0*2/3 + 2/3, 2/3*1 + 1/3*2) = (2/3, 4/3),
         lse = ln 3.
    Then move token 0's key to (1,0): A_2 = (1,0)(1,0)^T, m_2 = <q,k0> v0 = (1,0),
    y_2 = (2/3 + 3/4, 4/3)."""
    q = np.array([[1.0, 0.0]] * 3)
    k = np.array([[0.0, 0.0], [math.log(2.0), 0.0], [0.0, 5.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]])
    g = math.log(3.0)
    y, A, lse = fwd1(q, k, v, 1.0, 1.0, g, 2, scale=1.0)
    np.testing.assert_allclose(y, [[1, 0], [1 / 3, 2 / 3], [2 / 3, 4 / 3]], atol=1e-14)
    np.testing.assert_allclose(lse, [0.0, math.log(3.0), math.log(3.0)], atol=1e-14)
    np.testing.assert_allclose(A, np.zeros((2, 2)), atol=0)
    k[0] = [1.0, 0.0]
    y, A, lse = fwd1(q, k, v, 1.0, 1.0, g, 2, scale=1.0)
    np.testing.assert_allclose(y[2], [2 / 3 + 3 / 4, 4 / 3], atol=1e-14)
    np.testing.assert_allclose(A, [[1.0, 0.0], [0.0, 0.0]], atol=0)


# --------------------------------------------------------------------------- special cases


def sdpa_band(q, k, v, W, scale):
    """torch scaled_dot_product_attention (CPU, float64) with a band mask."""
    T = q.shape[0]
    mask = torch.from_numpy(dense.band_mask(T, W))
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))[None, None]  # noqa: E731
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask,
                                                            scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("T,D,W", [(40, 8, 5), (64, 16, 8), (9, 4, 1), (30, 3, 29)])
def test_gate_closed_is_sliding_window_attention(T, D, W):
    """sigma(g) -> 0: TC reduces to pure sliding-window softmax attention."""
    q, k, v = one_head(T, D, 11)
    y, _, _ = fwd1(q, k, v, 0.9, 0.5, -800.0, W)
    np.testing.assert_allclose(y, sdpa_band(q, k, v, W, 1 / math.sqrt(D)), rtol=1e-12, atol=1e-13)


def test_eta_zero_is_sliding_window_attention():
    q, k, v = one_head(50, 8, 12)
    y, A, _ = fwd1(q, k, v, 0.9, 0.0, 2.0, 6)
    np.testing.assert_allclose(y, sdpa_band(q, k, v, 6, 1 / math.sqrt(8)), rtol=1e-12, atol=1e-13)
    assert np.all(A == 0)


@pytest.mark.parametrize("T,W", [(20, 20), (20, 50), (1, 1), (7, 8)])
def test_full_window_is_causal_attention(T, W):
    """W >= T: no eviction, A = 0, plain causal softmax attention."""
    D = 8
    q, k, v = one_head(T, D, 13)
    y, A, _ = fwd1(q, k, v, 0.9, 0.5, 1.0, W)
    tt = lambda x: torch.from_numpy(x)[None, None]  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(tt(q), tt(k), tt(v), is_causal=True)[0, 0].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    assert np.all(A == 0)


def memory_part(q, k, v, lam, eta, W):
    g = 0.7
    sg = 1 / (1 + math.exp(-g))
    y, _, _ = fwd1(q, k, v, lam, eta, g, W)
    y0, _, _ = fwd1(q, k, v, lam, eta, -800.0, W)
    return (y - y0) / sg


def test_lambda_one_is_shifted_cumsum_linear_attention():
    """lam = 1: A_t = eta * cumsum_{i<=t-W} k_i v_i^T (numpy cumsum)."""
    T, D, W, eta = 30, 5, 4, 0.3
    q, k, v = one_head(T, D, 21)
    m = memory_part(q, k, v, 1.0, eta, W)
    outer = np.einsum("ia,ic->iac", k, v)
    cs = np.cumsum(outer, axis=0)
    for t in range(T):
        A = eta * cs[t - W] if t >= W else np.zeros((D, D))
        np.testing.assert_allclose(m[t], q[t] @ A, rtol=1e-9, atol=1e-11)


def test_lambda_zero_keeps_only_latest_eviction():
    """lam = 0 (0^0 = 1): A_t = eta k_{t-W} v_{t-W}^T."""
    T, D, W, eta = 25, 4, 3, 0.6
    q, k, v = one_head(T, D, 22)
    m = memory_part(q, k, v, 0.0, eta, W)
    for t in range(T):
        ref = eta * np.dot(q[t], k[t - W]) * v[t - W] if t >= W else np.zeros(D)
        np.testing.assert_allclose(m[t], ref, rtol=1e-10, atol=1e-12)


def test_partition_invariant_each_token_one_path():
    """Section 3.2: every prior token feeds exactly one read path.  With one-hot
    values v_i = e_i (T <= D) output coordinate i of y_t is token i's weight:
    a softmax weight for t-W < i <= t, sigma*eta*lam^(t-W-i)<q_t,k_i> for
    i <= t-W, and 0 for i > t."""
    T = D = 24
    W, lam, eta, g = 5, 0.8, 0.45, 0.3
    sg = 1 / (1 + math.exp(-g))
    q, k, _ = one_head(T, D, 23)
    v = np.eye(T)
    y, _, lse = fwd1(q, k, v, lam, eta, g, W)
    tau = 1 / math.sqrt(D)
    for t in range(T):
        for i in range(T):
            if i > t:
                ref = 0.0
            elif i > t - W:
                ref = math.exp(tau * np.dot(q[t], k[i]) - lse[t])
            else:
                ref = sg * eta * lam ** (t - W - i) * np.dot(q[t], k[i])
            assert abs(y[t, i] - ref) < 1e-12, (t, i)
        band = [i for i in range(T) if t - W < i <= t]
        assert abs(sum(y[t, i] for i in band) - 1.0) < 1e-12


@pytest.mark.parametrize("T,D,W,lam,eta,g", [(48, 8, 6, 0.9, 0.5, 0.0), (33, 4, 1, 0.5, 1.0, -1.0),
                                             (40, 16, 39, 0.99, 0.1, 2.0), (26, 5, 30, 0.7, 0.7, 0.5)])
def test_matches_dense_masked_form(T, D, W, lam, eta, g):
    """The read identity q(k outer v) = <q,k> v turns the layer into one dense
    masked T x T form (numpy matmul)."""
    q, k, v = one_head(T, D, 31)
    y, _, lse = fwd1(q, k, v, lam, eta, g, W)
    yd, lsed = dense.dense_forward(q, k, v, lam, eta, g, W, 1 / math.sqrt(D))
    np.testing.assert_allclose(y, yd, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=1e-12, atol=1e-12)


def test_batched_heads_use_their_own_parameters():
    B, H, T, D, W = 2, 3, 20, 4, 5
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    lam, eta, g = np.array([0.5, 0.9, 0.99]), np.array([0.1, 0.5, 1.0]), np.array([-1.0, 0.0, 1.0])
    y, A, lse = oracle.forward(q, k, v, lam, eta, g, W)
    for b in range(B):
        for h in range(H):
            y1, A1, l1 = fwd1(q[b, h], k[b, h], v[b, h], lam[h], eta[h], g[h], W)
            np.testing.assert_array_equal(y[b, h], y1)
            np.testing.assert_array_equal(A[b, h], A1)
            np.testing.assert_array_equal(lse[b, h], l1)


# --------------------------------------------------------------------------- scan claims


@pytest.mark.parametrize("lam", [0.881, 0.993])
def test_chunked_scan_equals_per_token_writes_fp32(lam):
    """Abstract / contributions: the parallel weighted-sum scan matches per-token
    writes to float32 rounding; the bar here is 1e-6 relative."""
    T, D, W, C, eta = 4096, 64, 256, 64, 0.3
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((T, D)).astype(np.float32) / 8 for _ in range(3))
    ms, As = oracle.memory_f32_sequential(q, k, v, lam, eta, W)
    mc, Ac = oracle.memory_f32_chunked(q, k, v, lam, eta, W, C)
    assert rel(mc, ms) < 1e-6
    assert rel(Ac, As) < 1e-6
    # and both are float32 roundings of the exact (float64) value
    m64 = memory_part(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                      np.float64(np.float32(lam)), np.float64(np.float32(eta)), W)
    assert rel(mc, m64) < 1e-6 and rel(ms, m64) < 1e-6


@pytest.mark.parametrize("C", [1, 3, 8, 64, 100, 5000])
def test_chunked_scan_result_independent_of_chunk(C):
    T, D, W = 300, 8, 17
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((T, D)).astype(np.float32) for _ in range(3))
    m1, A1 = oracle.memory_f32_sequential(q, k, v, 0.95, 0.4, W)
    mc, Ac = oracle.memory_f32_chunked(q, k, v, 0.95, 0.4, W, C)
    assert rel(mc, m1) < 2e-6 and rel(Ac, A1) < 2e-6


@pytest.mark.parametrize("C", [1, 2, 5, 8])
def test_chunk_mean_shortcut_adds_c2_minus_c_cross_terms(C):
    """Abstract: the chunk-mean write eta*(kbar outer vbar) differs from the
    per-token sum by exactly C^2 - C cross terms k_i outer v_j (i != j) per chunk
    (with the C^2 factor the mean introduces; lam = 1 within the chunk)."""
    D = 4
    rng = np.random.default_rng(C)
    kc, vc = rng.standard_normal((C, D)), rng.standard_normal((C, D))
    A0 = np.zeros((D, D))
    shortcut = dense.chunk_mean_write(A0, kc, vc, 1.0, 1.0)
    exact = sum(np.outer(kc[i], vc[i]) for i in range(C))
    cross = [np.outer(kc[i], vc[j]) for i in range(C) for j in range(C) if i != j]
    assert len(cross) == C * C - C
    diff = C * C * shortcut - exact
    np.testing.assert_allclose(diff, sum(cross) if cross else np.zeros((D, D)), atol=1e-12)
    # the per-token recurrence never forms those cross terms
    q = np.zeros((C + 1, D))
    kk = np.vstack([kc, np.zeros((1, D))])
    vv = np.vstack([vc, np.zeros((1, D))])
    _, A, _ = fwd1(np.vstack([q]), kk, vv, 1.0, 1.0, 0.0, 1)
    np.testing.assert_allclose(A, exact, atol=1e-12)


# --------------------------------------------------------------------------- decode


def test_decode_steps_reproduce_forward():
    """Figure 2 streaming steps from an empty ring equal the prefill recurrence,
    and forward(T+n) = forward(T) then n decode steps."""
    S, H, D, W, T = 2, 3, 4, 5, 23
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((S, H, T, D)) for _ in range(3))
    lam, eta, g = np.array([0.5, 0.9, 0.99]), np.array([0.2, 0.5, 0.9]), np.array([0.3, -0.2, 1.0])
    y, A, _ = oracle.forward(q, k, v, lam, eta, g, W)
    kr = np.zeros((S, H, W, D))
    vr = np.zeros((S, H, W, D))
    Ad = np.zeros((S, H, D, D))
    pos = np.zeros(S, np.int64)
    for t in range(T):
        yt = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], kr, vr, Ad, pos, lam, eta, g)
        np.testing.assert_allclose(yt, y[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Ad, A, rtol=1e-12, atol=1e-13)
    assert np.all(pos == T)
    # handoff: state of forward(T0) + ring of its last W pairs, then decode
    T0 = 14
    _, A0, _ = oracle.forward(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], lam, eta, g, W)
    kr = np.zeros((S, H, W, D))
    vr = np.zeros((S, H, W, D))
    for t in range(T0 - W, T0):
        kr[:, :, t % W] = k[:, :, t]
        vr[:, :, t % W] = v[:, :, t]
    pos = np.full(S, T0, np.int64)
    A0 = np.ascontiguousarray(A0)
    for t in range(T0, T):
        yt = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], kr, vr, A0, pos, lam, eta, g)
        np.testing.assert_allclose(yt, y[:, :, t], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cuts", [(0, 23), (0, 3, 23), (0, 5, 6, 17, 23), (0, 11, 12, 23)])
def test_continuation_in_chunks_reproduces_forward(cuts):
    """Chunked continuation (each chunk T successive streaming steps from the
    ring and memory the previous chunk left) equals one forward over the
    whole sequence, whatever the chunk boundaries (before, at and after the
    first eviction at t = W)."""
    B, H, D, W, T = 2, 3, 4, 5, 23
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    lam, eta, g = np.array([0.5, 0.9, 0.99]), np.array([0.2, 0.5, 0.9]), np.array([0.3, -0.2, 1.0])
    y, A, _ = oracle.forward(q, k, v, lam, eta, g, W)
    kr, vr, Ad = np.zeros((B, H, W, D)), np.zeros((B, H, W, D)), np.zeros((B, H, D, D))
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(oracle.forward_continue(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], kr, vr, Ad, a,
                                             lam, eta, g))
    np.testing.assert_allclose(np.concatenate(parts, axis=2), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Ad, A, rtol=1e-12, atol=1e-13)
    for t in range(T - W, T):  # the ring holds the last W pairs at slot t mod W
        assert np.array_equal(kr[:, :, t % W], k[:, :, t]) and np.array_equal(vr[:, :, t % W], v[:, :, t])


def test_state_after_writes_matches_recurrence():
    rng = np.random.default_rng(10)
    n, D = 40, 6
    k, v = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    q = np.zeros((n + 1, D))
    kk = np.vstack([k, np.zeros((1, D))])
    vv = np.vstack([v, np.zeros((1, D))])
    _, A, _ = fwd1(q, kk, vv, 0.93, 0.37, 0.0, 1)
    np.testing.assert_allclose(dense.state_after_writes(k, v, 0.93, 0.37), A, rtol=1e-12, atol=1e-13)


def test_capacity_probe_reads_gram_weighted_values():
    """The capacity probe (window 1, lambda = eta = 1, N write pairs then N
    reads with the stored keys) reads y_{N+i} = sigmoid(g) sum_j <k_i,k_j> v_j:
    the Gram matrix of the keys times the values (q (k outer v) = <q,k> v
    summed over the memory).  With orthonormal keys every value comes back
    exactly."""
    import tc_inputs

    for N, D, ortho in [(24, 16, False), (16, 16, True), (5, 8, True)]:
        q, k, v, lam, eta, g, vals = tc_inputs.capacity_inputs(N, D, H=2, dtype="f32", orthonormal=ortho)
        y, A, _ = oracle.forward(q, k, v, lam, eta, g, 1)
        keys = k[0, :, :N].astype(np.float64)
        sg = 1.0 / (1.0 + np.exp(-30.0))
        want = sg * np.einsum("hij,hjd->hid", keys @ keys.transpose(0, 2, 1), vals.astype(np.float64))
        np.testing.assert_allclose(y[0, :, N:], want, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(A[0], np.einsum("hja,hjc->hac", keys, vals.astype(np.float64)), rtol=1e-12,
                                   atol=1e-13)
        if ortho:
            np.testing.assert_allclose(y[0, :, N:], vals, rtol=0, atol=1e-5)

