"""Pins of the oracle's backward pass (gradients of L = sum_t <dy_t, y_t> with
respect to q, k, v and the per-head lambda, eta, g, which the abstract says
are trained end to end).

Pinned by (1) central finite differences of the oracle's own forward in
float64, (2) torch autograd (CPU, float64) of an independently written dense
masked form of the layer, and (3) exact homogeneity (Euler) identities of the
memory path.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def case(seed, B=1, H=2, T=24, D=4, W=5):
    rng = np.random.default_rng(seed)
    q, k, v, dy = (rng.standard_normal((B, H, T, D)) for _ in range(4))
    lam = rng.uniform(0.5, 0.97, H)
    eta = rng.uniform(0.1, 0.9, H)
    g = rng.standard_normal(H)
    return q, k, v, dy, lam, eta, g, W


def loss(q, k, v, dy, lam, eta, g, W):
    y, _, _ = oracle.forward(q, k, v, lam, eta, g, W)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("seed,W", [(0, 5), (1, 1), (2, 11), (3, 30)])
def test_backward_matches_finite_differences(seed, W):
    q, k, v, dy, lam, eta, g, _ = case(seed, W=W)
    dq, dk, dv, dl, de, dg = oracle.backward(q, k, v, dy, lam, eta, g, W)
    rng = np.random.default_rng(100 + seed)
    h = 1e-5
    args = dict(q=q, k=k, v=v, lam=lam, eta=eta, g=g)
    grads = dict(q=dq, k=dk, v=dv, lam=dl, eta=de, g=dg)
    for name in ["q", "k", "v"]:
        for _ in range(3):
            d = rng.standard_normal(args[name].shape)
            a1 = dict(args)
            a2 = dict(args)
            a1[name] = args[name] + h * d
            a2[name] = args[name] - h * d
            fd = (loss(a1["q"], a1["k"], a1["v"], dy, a1["lam"], a1["eta"], a1["g"], W)
                  - loss(a2["q"], a2["k"], a2["v"], dy, a2["lam"], a2["eta"], a2["g"], W)) / (2 * h)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    for name in ["lam", "eta", "g"]:
        for hh in range(len(lam)):
            a1 = dict(args)
            a2 = dict(args)
            a1[name] = args[name].copy()
            a2[name] = args[name].copy()
            a1[name][hh] += h
            a2[name][hh] -= h
            fd = (loss(a1["q"], a1["k"], a1["v"], dy, a1["lam"], a1["eta"], a1["g"], W)
                  - loss(a2["q"], a2["k"], a2["v"], dy, a2["lam"], a2["eta"], a2["g"], W)) / (2 * h)
            an = grads[name][hh]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, hh, fd, an)


def torch_dense_layer(q, k, v, lam, eta, g, W):
    """Independent dense form in torch: band softmax plus masked decayed
    linear attention (read identity), [B,H,T,D] float64."""
    T = q.shape[2]
    D = q.shape[3]
    t = torch.arange(T)[:, None]
    i = torch.arange(T)[None, :]
    band = (i <= t) & (i > t - W)
    lag = (t - W - i).to(torch.float64)
    memmask = lag >= 0
    Z = q @ k.transpose(-1, -2)
    S = torch.where(band, Z / math.sqrt(D), torch.tensor(-math.inf, dtype=torch.float64))
    P = torch.softmax(S, dim=-1)
    lamh = lam[:, None, None]
    L = torch.where(memmask, eta[:, None, None] * lamh ** torch.clamp(lag, min=0.0),
                    torch.zeros((), dtype=torch.float64))
    return P @ v + torch.sigmoid(g)[:, None, None] * ((Z * L) @ v)


@pytest.mark.parametrize("seed,W", [(4, 5), (5, 2), (6, 13)])
def test_backward_matches_torch_autograd_of_dense_form(seed, W):
    q, k, v, dy, lam, eta, g, _ = case(seed, B=2, H=2, T=20, D=3, W=W)
    dq, dk, dv, dl, de, dg = oracle.backward(q, k, v, dy, lam, eta, g, W)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tl, te, tg = (torch.tensor(x, requires_grad=True) for x in (lam, eta, g))
    y = torch_dense_layer(tq, tk, tv, tl, te, tg, W)
    (y * torch.tensor(dy)).sum().backward()
    for a, b in [(dq, tq), (dk, tk), (dv, tv), (dl, tl), (de, te), (dg, tg)]:
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_memory_path_euler_identities():
    """m_t is linear in q, in k (through every write), in v, and in eta, so
    <q,dq_L2> = <k,dk_L2> = <v,dv_L2> = eta*deta = sum_t <dm_t, m_t>; and
    dg = sigma(1-sigma) sum_t <dy_t, m_t>.  The L2 parts are the difference
    between the full gradient and the gate-closed (sigma=0) gradient."""
    q, k, v, dy, lam, eta, g, W = case(7, B=1, H=1, T=30, D=5, W=4)
    full = oracle.backward(q, k, v, dy, lam, eta, g, W)
    l1 = oracle.backward(q, k, v, dy, lam, eta, np.array([-800.0]), W)
    dq2, dk2, dv2 = (full[i] - l1[i] for i in range(3))
    sg = 1 / (1 + math.exp(-g[0]))
    y, _, _ = oracle.forward(q, k, v, lam, eta, g, W)
    y0, _, _ = oracle.forward(q, k, v, lam, eta, np.array([-800.0]), W)
    m = (y - y0) / sg
    s = float(np.sum(sg * dy * m))
    for val in [np.sum(q * dq2), np.sum(k * dk2), np.sum(v * dv2), eta[0] * full[4][0]]:
        assert abs(val - s) < 1e-10 * max(1, abs(s))
    assert abs(full[5][0] - sg * (1 - sg) * np.sum(dy * m)) < 1e-11
