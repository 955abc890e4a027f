"""The raw memory-capacity probe on the GPU (window 1, lambda = eta = 1: N
write pairs, then N reads with the stored keys) against the CPU oracle, through
both the forward and the decode step: the same reads, and the same recall."""
import numpy as np
import pytest
import torch

import oracle
import tc_inputs
from gpu_util import TOL, dev, host, rel, say

pytestmark = pytest.mark.gpu


def tc():
    import eviction_fed_weight_amd as m

    return m


def recall(reads, vals):
    r = reads / np.linalg.norm(reads, axis=-1, keepdims=True)
    s = vals / np.linalg.norm(vals, axis=-1, keepdims=True)
    hits = np.argmax(np.einsum("hid,hjd->hij", r, s), axis=-1) == np.arange(vals.shape[1])
    return hits.mean()


@pytest.mark.parametrize("N,D", [(16, 64), (64, 64), (256, 64), (1024, 64), (200, 128)])
def test_capacity_probe_forward(N, D):
    say("capacity forward", N, D)
    q, k, v, lam, eta, g, vals = tc_inputs.capacity_inputs(N, D, H=3)
    y, _, _ = tc().tc_forward(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(lam), dev(eta), dev(g), 1)
    torch.cuda.synchronize()
    yo, _, _ = oracle.forward(q, k, v, lam, eta, g, 1)
    reads, reads_o = host(y)[0, :, N:], yo[0, :, N:]
    e = rel(reads, reads_o)
    rg, ro = recall(reads, vals), recall(reads_o, vals)
    say("  rel", e, "recall gpu", rg, "oracle", ro)
    assert e <= TOL["bf16"]
    assert abs(rg - ro) <= 2.0 / N  # a near-tie may resolve either way


def test_capacity_probe_decode_steps():
    """The same probe streamed through tc_decode_step (each step evicts the
    previous token into A): reads match the forward's."""
    N, D, H = 48, 64, 2
    q, k, v, lam, eta, g, vals = tc_inputs.capacity_inputs(N, D, H=H)
    L, E, G = dev(lam), dev(eta), dev(g)
    kr = torch.zeros((1, H, 1, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    A = torch.zeros((1, H, D, D), dtype=torch.float32, device="cuda")
    pos = torch.zeros(1, dtype=torch.int64, device="cuda")
    ys = []
    for t in range(2 * N):
        ys.append(host(tc().tc_decode_step(dev(q[:, :, t], "bf16"), dev(k[:, :, t], "bf16"), dev(v[:, :, t], "bf16"),
                                           kr, vr, A, pos, L, E, G)))
    torch.cuda.synchronize()
    reads = np.stack(ys, axis=2)[0, :, N:]
    yo, _, _ = oracle.forward(q, k, v, lam, eta, g, 1)
    assert rel(reads, yo[0, :, N:]) <= TOL["bf16"]
    assert abs(recall(reads, vals) - recall(yo[0, :, N:], vals)) <= 2.0 / N
