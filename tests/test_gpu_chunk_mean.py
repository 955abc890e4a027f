"""GPU parity of tc_forward_chunk_mean, the chunk-mean shortcut (one write
A <- lam A + eta kbar vbar^T per chunk of C evicted pairs, the ablation the
abstract and Section 1 of "Tensor Cache: Eviction-conditioned Associative
Memory for Transformers" compare the exact scan with), through the C ABI,
against the oracle's forward_chunk_mean; and its distance from the exact
scan on the same inputs, which must be that of the two oracles."""
import numpy as np
import pytest
import torch

import oracle
import tc_inputs
from gpu_util import bar, dev, errors, host, rel, say

pytestmark = pytest.mark.gpu


def tc():
    import eviction_fed_weight_amd as m

    return m


def compare(d, W, C, heads=None):
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    y, A, lse = tc().tc_forward_chunk_mean(q, k, v, lam, eta, g, W, C)
    torch.cuda.synchronize()
    y, A, lse = host(y), host(A), host(lse)
    err = {}
    for b, h in heads or [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]:
        sl = lambda x: x[b:b + 1, h:h + 1]  # noqa: E731
        yo, Ao, lo = oracle.forward_chunk_mean(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["lam"][h:h + 1],
                                               d["eta"][h:h + 1], d["gate"][h:h + 1], W, C)
        for key, e in errors(y=(sl(y), yo), A=(sl(A), Ao), lse=(sl(lse), lo)).items():
            err[key] = max(err.get(key, 0.0), e)
    return err


CASES = [
    # B, H, T, D, W, C
    (2, 2, 500, 64, 128, 64),      # one segment: the carry of 64-chunks inside the workgroup, ragged end
    (1, 2, 700, 64, 256, 128),     # 128-chunks, last chunk incomplete (not in A_final)
    (2, 3, 333, 32, 128, 64),      # D = 32
    (1, 2, 300, 16, 64, 64),       # D = 16, a block whose first chunk is before token 0
    (1, 1, 200, 64, 256, 128),     # T < W: the sliding window alone, A = 0
    (1, 2, 64 * 140, 64, 256, 64),  # 70 one-block segments: state pass and chain kernel
    (4, 64, 1024 + 37, 64, 256, 128),  # several blocks per segment (sampled heads below)
]


@pytest.mark.parametrize("B,H,T,D,W,C", CASES)
def test_chunk_mean_matches_the_oracle(B, H, T, D, W, C):
    say("chunk mean", B, H, T, D, W, C)
    d = tc_inputs.prefill_inputs(2, seed=101 + T + C, B=B, H=H, T=T, D=D, W=W, dtype="bf16", plants=False)
    heads = [(0, 0), (1, 33), (3, 63)] if B * H > 16 else None
    err = compare(d, W, C, heads)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_chunk_mean_training_shape_full():
    """The training-shape prefill (B=8 H=8 T=1024 W=256) with its C = 64."""
    d = tc_inputs.prefill_inputs(2)
    err = compare(d, 256, 64)
    say("chunk mean, training shape", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_chunk_mean_long_prefill_sampled_heads_and_gap_to_the_exact_scan():
    """The long-context prefill (C = 128): the shortcut matches its oracle on
    two whole heads, and its relative distance from the exact scan's output
    equals the two oracles' distance (the gap is the method's, not rounding)."""
    d = tc_inputs.prefill_inputs(3)
    m = tc()
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    ys, _, _ = m.tc_forward_chunk_mean(q, k, v, lam, eta, g, 1024, 128)
    ye, _, _ = m.tc_forward(q, k, v, lam, eta, g, 1024, 128)
    torch.cuda.synchronize()
    ys, ye = host(ys), host(ye)
    for h in (0, 7):
        sl = lambda x: x[:, h:h + 1]  # noqa: E731
        yso, _, _ = oracle.forward_chunk_mean(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["lam"][h:h + 1],
                                              d["eta"][h:h + 1], d["gate"][h:h + 1], 1024, 128)
        yeo, _, _ = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["lam"][h:h + 1], d["eta"][h:h + 1],
                                   d["gate"][h:h + 1], 1024)
        err = errors(y=(sl(ys), yso))
        gap_gpu, gap_oracle = rel(sl(ys), sl(ye)), rel(yso, yeo)
        say("  head", h, err, "gap", gap_gpu, "oracle gap", gap_oracle)
        for key, e in err.items():
            assert e <= bar(key, "bf16"), (h, key, e)
        assert gap_oracle > 1e-2  # the shortcut is a different function, not a rounding of the exact one
        assert abs(gap_gpu - gap_oracle) <= 5e-3 * (1 + gap_oracle)


def test_chunk_mean_refuses_what_it_does_not_build():
    m = tc()
    d = tc_inputs.prefill_inputs(2, seed=7, B=1, H=1, T=300, D=64, W=128, dtype="bf16", plants=False)
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    for W, C in ((128, 32), (100, 64), (192, 128)):
        with pytest.raises(m.TCError) as e:
            m.tc_forward_chunk_mean(q, k, v, lam, eta, g, W, C)
        assert e.value.status == m.TC_ERR_UNSUPPORTED, (W, C)
    with pytest.raises(m.TCError) as e:
        m.tc_forward_chunk_mean(q.float(), k.float(), v.float(), lam, eta, g, 128, 64)
    assert e.value.status == m.TC_ERR_UNSUPPORTED
