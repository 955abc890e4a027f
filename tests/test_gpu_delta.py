"""GPU parity of tc_forward_delta, the layer with the delta-rule write (the
optional write of Figure 2, step 3, of "Tensor Cache: Eviction-conditioned
Associative Memory for Transformers"; reading: the evicted key's prediction
error u = v_old - k_old A is written, A <- lam A + eta k_old u^T), through
the C ABI, against the oracle's per-token forward_delta.

Inputs are drawn as the training-shape prefill draws them (q, k, v ~
N(0,1)/8 stored in the tested dtype, lam = sigmoid(U(2,5)), eta =
sigmoid(U(-3,0)), g ~ N(0,1)): with keys of norm about one the write is a
contraction (eta |k|^2 < 2), as the delta rule needs."""
import numpy as np
import pytest
import torch

import oracle
import tc_inputs
from gpu_util import bar, dev, errors, host, say

pytestmark = pytest.mark.gpu


def tc():
    import eviction_fed_weight_amd as m

    return m


def compare(d, W, dtype, heads=None):
    q, k, v = (dev(d[x], dtype) for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    y, A, lse = tc().tc_forward_delta(q, k, v, lam, eta, g, W)
    torch.cuda.synchronize()
    y, A, lse = host(y), host(A), host(lse)
    err = {}
    for b, h in heads or [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]:
        sl = lambda x: x[b:b + 1, h:h + 1]  # noqa: E731
        yo, Ao, lo = oracle.forward_delta(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["lam"][h:h + 1], d["eta"][h:h + 1],
                                          d["gate"][h:h + 1], W)
        for key, e in errors(y=(sl(y), yo), A=(sl(A), Ao), lse=(sl(lse), lo)).items():
            err[key] = max(err.get(key, 0.0), e)
    return err


CASES = [
    # B, H, T, D, W, dtype
    (1, 1, 64, 16, 8, "f32"),      # one incomplete chunk of 56 writes
    (1, 2, 700, 64, 100, "f32"),   # ten chunks, the last of 24 writes
    (2, 2, 333, 32, 40, "bf16"),   # D = 32, ragged
    (2, 3, 1000, 64, 256, "bf16"),
    (1, 2, 600, 128, 64, "bf16"),  # D = 128: eight chunks, rows of the last past T
    (1, 1, 450, 128, 100, "f32"),  # float32 D = 128
    (2, 2, 300, 16, 64, "bf16"),   # D = 16
    (1, 2, 200, 64, 256, "bf16"),  # T < W: no write, the window alone
    (1, 1, 64 + 64, 64, 64, "bf16"),  # exactly one full chunk
    (1, 2, 64 * 100 + 300, 64, 256, "bf16"),  # 101 chunks: 34 groups of 3 (the last of 2) in 12 supergroups of 3 (the last of 1)
    (1, 1, 64 * 40 + 100, 128, 128, "bf16"),  # D = 128, 40 chunks in groups of 4
    (1, 1, 64 * 20 + 30, 32, 64, "f32"),      # float32, 20 chunks in groups of 2
    (1, 1, 64 * 169 + 20 + 128, 64, 128, "f32"),  # float32, 170 chunks: 43 groups of 4 (the last of 2) in 11 supergroups of 4 (the last of 3)
    (1, 1, 64 * 256 + 10 + 128, 64, 128, "f32"),  # float32, 257 chunks: 65 groups of 4 (the last of 1) in 13 supergroups of 5
    (1, 2, 64 * 96 + 1 + 64, 32, 64, "bf16"),     # D = 32, 97 chunks: 33 groups of 3 (the last of 1) in 11 supergroups of 3
    (1, 3, 64 * 149 + 33 + 100, 16, 100, "f32"),  # D = 16, 150 chunks: 50 groups of 3 in 13 supergroups of 4 (the last of 2)
]


@pytest.mark.parametrize("B,H,T,D,W,dtype", CASES)
def test_delta_matches_the_oracle(B, H, T, D, W, dtype):
    say("delta", B, H, T, D, W, dtype)
    d = tc_inputs.prefill_inputs(2, seed=303 + T + D, B=B, H=H, T=T, D=D, W=W, dtype=dtype, plants=False)
    err = compare(d, W, dtype)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, dtype), (key, e)


def test_delta_training_shape_full():
    """The training-shape prefill (B=8 H=8 T=1024 W=256 D=64 bf16), every head."""
    d = tc_inputs.prefill_inputs(2)
    err = compare(d, 256, "bf16")
    say("delta, training shape", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_delta_differs_from_the_outer_product_write():
    """On the same inputs the two writes give different memories (the
    correction term is live), and the delta layer's memory stays bounded."""
    d = tc_inputs.prefill_inputs(2, seed=9, B=1, H=2, T=800, D=64, W=128, dtype="bf16", plants=False)
    m = tc()
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    _, A1, _ = m.tc_forward_delta(q, k, v, lam, eta, g, 128)
    _, A0, _ = m.tc_forward(q, k, v, lam, eta, g, 128)
    A1, A0 = host(A1), host(A0)
    assert np.isfinite(A1).all()
    assert np.linalg.norm(A1 - A0) > 1e-2 * np.linalg.norm(A0)
