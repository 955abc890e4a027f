"""tc_forward_noalloc (the forward for callers that cannot allocate) through
the C ABI, against tc_forward on the same inputs: two calls in a row, the
second with a smaller shape, each bit-identical to tc_forward's outputs (the
same kernels and plan, only the workspace differs) and within the parity
bars of the oracle; a shape whose workspace exceeds the 32 MiB scratch is
refused before anything runs."""
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


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_tc_forward_twice(order):
    m = tc()
    cases = [dict(B=8, H=8, T=1024, D=64, W=256, seed=91),   # the training-shape prefill: state exchange, 9.4 MB
             dict(B=2, H=3, T=700, D=64, W=100, seed=92)]    # smaller: fewer segments, the earlier call's data left behind
    for c in cases:
        say("noalloc", c)
        d = tc_inputs.prefill_inputs(2, seed=c["seed"], B=c["B"], H=c["H"], T=c["T"], D=c["D"], W=c["W"],
                                     dtype="bf16", plants=False)
        q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
        lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
        shape = m.make_shape(c["B"], c["H"], c["T"], c["D"], c["W"], 64, 0.0, m.TC_BF16)
        assert m.tc_forward_workspace_size(shape) <= m.NOALLOC_SCRATCH_BYTES
        y0, A0, l0 = m.tc_forward(q, k, v, lam, eta, g, c["W"])
        y = torch.empty_like(q)
        A = torch.empty_like(A0)
        lse = torch.empty_like(l0)
        m.tc_forward_noalloc(q, k, v, lam, eta, g, c["W"], y=y, A_final=A, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(A, A0) and torch.equal(lse, l0)
        yo, Ao, lo = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], c["W"])
        err = errors(y=(host(y), yo), A=(host(A), Ao), lse=(host(lse), lo))
        say("  errors", err)
        for key, e in err.items():
            assert e <= bar(key, "bf16"), (key, e)


def test_noalloc_refuses_a_shape_beyond_the_scratch():
    m = tc()
    B, H, T, D, W = 16, 32, 2048, 64, 256
    shape = m.make_shape(B, H, T, D, W, 64, 0.0, m.TC_BF16)
    assert m.tc_forward_workspace_size(shape) > m.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(H, device="cuda")
    y = torch.full_like(q, 7.0)
    with pytest.raises(m.TCError) as e:
        m.tc_forward_noalloc(q, q, q, p, p, p, W, y=y)
    assert e.value.status == m.TC_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing ran
