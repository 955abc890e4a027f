"""GPU parity of tc_forward_continue (chunked prefill after earlier tokens and
the prefill -> decode handoff, through the C ABI) against the CPU oracle.

The oracle of a continuation is its definition: T successive streaming steps
(Figure 2) from the ring and memory handed in (oracle.forward_continue); the
softmax normaliser is compared with the oracle forward over the whole
sequence (it does not depend on the memory)."""
import numpy as np
import pytest
import torch

import oracle
import tc_inputs
from gpu_util import TOL, bar, dev, errors, host, rel, say

pytestmark = pytest.mark.gpu


def tc():
    import eviction_fed_weight_amd as m

    return m


def sequence(seed, B, H, T, D, dtype):
    rng = np.random.default_rng(seed)
    x = [(rng.standard_normal((B, H, T, D)) / np.sqrt(D)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        x = [tc_inputs.bf16_round(a) for a in x]
    lam, eta, g = tc_inputs.head_params(rng, rng, rng, H)
    return x, lam, eta, g


def state_at(q, k, v, lam, eta, g, T0, W):
    """Ring (slot t mod W, other slots zero) and float32 memory after T0 tokens."""
    B, H, _, D = q.shape
    kr, vr = np.zeros((B, H, W, D)), np.zeros((B, H, W, D))
    for t in range(max(0, T0 - W), T0):
        kr[:, :, t % W] = k[:, :, t]
        vr[:, :, t % W] = v[:, :, t]
    if T0 > 0:
        _, A0, _ = oracle.forward(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], lam, eta, g, W)
    else:
        A0 = np.zeros((B, H, D, D))
    return kr, vr, A0.astype(np.float32).astype(np.float64)


CASES = [
    # B, H, T0 (tokens seen), T1 (new), D, W, dtype
    (1, 2, 0, 200, 16, 8, "f32"),        # fresh sequence: tc_forward plus the ring
    (2, 2, 5, 60, 16, 8, "f32"),         # pos0 < W
    (1, 2, 8, 70, 16, 8, "f32"),         # pos0 = W (first eviction is the first new token's)
    (2, 2, 150, 90, 64, 100, "f32"),     # pos0 > W, W not a multiple of the block
    (2, 2, 300, 333, 64, 128, "bf16"),   # 128-row kernel, several blocks, ragged tail
    (1, 3, 1000, 700, 64, 256, "bf16"),
    (1, 2, 600, 50, 64, 256, "bf16"),    # fewer new tokens than W
    (1, 2, 700, 300, 128, 128, "bf16"),  # D = 128
    (2, 1, 40, 1, 64, 64, "bf16"),       # one token: a decode step
    (1, 2, 70, 20, 32, 100, "bf16"),     # pos0 + T < W: no eviction at all
    (1, 2, 3000, 2500, 64, 1024, "bf16"),
    (1, 2, 300, 200, 64, 100, "bf16"),   # 128-row kernel, W not a multiple of the block (prefix 100 rows)
    (2, 2, 50, 70, 16, 32, "bf16"),      # D = 16 bf16
    (1, 1, 600, 150, 128, 256, "f32"),   # float32 D = 128
]


@pytest.mark.parametrize("B,H,T0,T1,D,W,dtype", CASES)
def test_continue_matches_streaming_steps(B, H, T0, T1, D, W, dtype):
    say("continue", B, H, T0, T1, D, W, dtype)
    (q, k, v), lam, eta, g = sequence(T0 * 7 + T1 + D, B, H, T0 + T1, D, dtype)
    kr, vr, A0 = state_at(q, k, v, lam, eta, g, T0, W)
    # oracle: T1 streaming steps from the same ring and (float32) memory
    okr, ovr, oA = kr.copy(), vr.copy(), A0.copy()
    sl = slice(T0, T0 + T1)
    yo = oracle.forward_continue(q[:, :, sl], k[:, :, sl], v[:, :, sl], okr, ovr, oA, T0, lam, eta, g)
    _, _, lo = oracle.forward(q, k, v, lam, eta, g, W)
    # GPU
    gk, gv, gA = dev(kr, dtype), dev(vr, dtype), dev(A0, "f32")
    pos = torch.full((B,), -1, dtype=torch.int64, device="cuda")
    Lm, Et, Gt = dev(lam), dev(eta), dev(g)
    y, lse = tc().tc_forward_continue(dev(q[:, :, sl], dtype), dev(k[:, :, sl], dtype), dev(v[:, :, sl], dtype),
                                      Lm, Et, Gt, gk, gv, gA, T0, pos=pos)
    torch.cuda.synchronize()
    err = errors(y=(host(y), yo), A=(host(gA), oA), lse=(host(lse), lo[:, :, sl]))
    say("  ", err)
    for name, e in err.items():
        assert e <= bar(name, dtype), (name, e)
    assert np.array_equal(host(gk), okr) and np.array_equal(host(gv), ovr)
    assert np.all(pos.cpu().numpy() == T0 + T1)


def test_continue_chunks_then_decode_equal_one_forward():
    """Prefill in three chunks (the first from an empty state), then decode
    steps from the ring and memory they leave: the whole stream equals one
    forward over the concatenated sequence."""
    B, H, D, W, dtype = 2, 2, 64, 256, "bf16"
    cuts = [0, 300, 301, 900]
    n_dec = 40
    T = cuts[-1] + n_dec
    say("chunks", cuts, "decode", n_dec)
    (q, k, v), lam, eta, g = sequence(77, B, H, T, D, dtype)
    yo, Ao, _ = oracle.forward(q, k, v, lam, eta, g, W)
    Lm, Et, Gt = dev(lam), dev(eta), dev(g)
    tdt = torch.bfloat16
    kr = torch.zeros((B, H, W, D), dtype=tdt, device="cuda")
    vr = torch.zeros_like(kr)
    A = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    ys = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        y, _ = tc().tc_forward_continue(dev(q[:, :, a:b], dtype), dev(k[:, :, a:b], dtype), dev(v[:, :, a:b], dtype),
                                        Lm, Et, Gt, kr, vr, A, a, pos=pos)
        ys.append(host(y))
    for t in range(cuts[-1], T):
        y = tc().tc_decode_step(dev(q[:, :, t], dtype), dev(k[:, :, t], dtype), dev(v[:, :, t], dtype),
                                kr, vr, A, pos, Lm, Et, Gt)
        ys.append(host(y)[:, :, None])
    torch.cuda.synchronize()
    err = errors(y=(np.concatenate(ys, axis=2), yo), A=(host(A), Ao))
    say("  ", err)
    for name, e in err.items():
        assert e <= bar(name, dtype), (name, e)
    assert np.all(pos.cpu().numpy() == T)


def test_continue_from_zero_equals_forward():
    """pos0 = 0: the continuation's outputs are tc_forward's (same kernels on
    the same rows) and its ring holds the last W tokens."""
    B, H, T, D, W, dtype = 1, 2, 700, 64, 256, "bf16"
    (q, k, v), lam, eta, g = sequence(5, B, H, T, D, dtype)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    Lm, Et, Gt = dev(lam), dev(eta), dev(g)
    y0, A0, l0 = tc().tc_forward(Q, K, V, Lm, Et, Gt, W)
    kr = torch.zeros((B, H, W, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    A = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    y1, l1 = tc().tc_forward_continue(Q, K, V, Lm, Et, Gt, kr, vr, A, 0)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(l0, l1)
    assert rel(host(A), host(A0)) <= 1e-6
    for t in range(T - W, T):
        assert torch.equal(kr[:, :, t % W], K[:, :, t]) and torch.equal(vr[:, :, t % W], V[:, :, t])


def test_continue_rejects_bad_arguments():
    B, H, T, D, W = 1, 1, 16, 64, 32
    x = torch.zeros((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros((B, H, W, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    A = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    p = torch.ones(H, dtype=torch.float32, device="cuda")
    with pytest.raises(tc().TCError):  # negative position
        tc().tc_forward_continue(x, x, x, p, p, p, kr, vr, A, -1)
    with pytest.raises(tc().TCError):  # the output ring aliases the input keys
        tc().tc_forward_continue(x, kr[:, :, :T], x, p, p, p, kr, vr, A, 4)


def test_continue_graph_capture():
    """tc_forward_continue captured in a HIP graph (pos0 is part of the
    captured call) and replayed from restored states on changed inputs, with
    an eager call between the replays: every replay matches the streaming-step
    oracle.  (No memset nodes; the forward takes its capture-safe path.)"""
    B, H, T0, T1, D, W, dtype = 1, 2, 700, 300, 64, 256, "bf16"
    m = tc()
    seqs = [sequence(90 + i, B, H, T0 + T1, D, dtype) for i in range(3)]
    sl = slice(T0, T0 + T1)
    states = [state_at(*x[0], *x[1:], T0, W) for x in seqs]
    q, k, v = (dev(seqs[0][0][j][:, :, sl], dtype) for j in range(3))
    lam, eta, g = (dev(x) for x in seqs[0][1:])
    kr, vr, A = dev(states[0][0], dtype), dev(states[0][1], dtype), dev(states[0][2], "f32")
    y = torch.empty_like(q)
    lse = torch.empty((B, H, T1), dtype=torch.float32, device="cuda")
    shape = m.make_shape(B, H, T1, D, W, 64, 0.0, m.TC_BF16)
    ws = torch.empty(m.tc_continue_workspace_size(shape, T0), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.tc_forward_continue(q, k, v, lam, eta, g, kr, vr, A, T0, y=y, lse=lse, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.tc_forward_continue(q, k, v, lam, eta, g, kr, vr, A, T0, y=y, lse=lse, ws=ws)
    torch.cuda.synchronize()
    for i in (1, 2, 0):
        (qq, kk, vv), la, et, ga = seqs[i]
        okr, ovr, oA = (x.copy() for x in states[i])
        yo = oracle.forward_continue(qq[:, :, sl], kk[:, :, sl], vv[:, :, sl], okr, ovr, oA, T0, la, et, ga)
        for dst, x in ((q, qq), (k, kk), (v, vv)):
            dst.copy_(dev(x[:, :, sl], dtype))
        for dst, x in ((lam, la), (eta, et), (g, ga)):
            dst.copy_(dev(x))
        for dst, x, dt in ((kr, states[i][0], dtype), (vr, states[i][1], dtype), (A, states[i][2], "f32")):
            dst.copy_(dev(x, dt))
        graph.replay()
        torch.cuda.synchronize()
        err = errors(y=(host(y), yo), A=(host(A), oA))
        say("  replay", i, err)
        for name, e in err.items():
            assert e <= bar(name, dtype), ("replay", i, name, e)
        assert np.array_equal(host(kr), okr)
        # an eager call from the same restored state on the same workspace
        for dst, x, dt in ((kr, states[i][0], dtype), (vr, states[i][1], dtype), (A, states[i][2], "f32")):
            dst.copy_(dev(x, dt))
        ye, _ = m.tc_forward_continue(q, k, v, lam, eta, g, kr, vr, A, T0, ws=ws)
        torch.cuda.synchronize()
        for name, e in errors(y=(host(ye), yo)).items():
            assert e <= bar(name, dtype), ("eager", i, name, e)



def test_continue_from_a_late_position_with_a_given_memory():
    """pos0 = 10^12 + 7 (slot and decay counts in 64-bit) and an arbitrary
    memory handed in: the ring holds the last W tokens at slot position mod W
    (ring order != time order), and the result equals the streaming steps."""
    B, H, T1, D, W, dtype = 2, 2, 300, 64, 128, "bf16"
    pos0 = 10 ** 12 + 7
    rng = np.random.default_rng(21)
    (q, k, v), lam, eta, g = sequence(22, B, H, W + T1, D, dtype)  # tokens pos0-W .. pos0+T1-1
    kr, vr = np.zeros((B, H, W, D)), np.zeros((B, H, W, D))
    for i in range(W):
        kr[:, :, (pos0 - W + i) % W] = k[:, :, i]
        vr[:, :, (pos0 - W + i) % W] = v[:, :, i]
    A0 = (rng.standard_normal((B, H, D, D)) * 0.3).astype(np.float32).astype(np.float64)
    okr, ovr, oA = kr.copy(), vr.copy(), A0.copy()
    sl = slice(W, W + T1)
    yo = oracle.forward_continue(q[:, :, sl], k[:, :, sl], v[:, :, sl], okr, ovr, oA, pos0, lam, eta, g)
    _, _, lo = oracle.forward(q, k, v, lam, eta, g, W)  # the window rows see only the ring and the new tokens
    gk, gv, gA = dev(kr, dtype), dev(vr, dtype), dev(A0, "f32")
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    y, lse = tc().tc_forward_continue(dev(q[:, :, sl], dtype), dev(k[:, :, sl], dtype), dev(v[:, :, sl], dtype),
                                      dev(lam), dev(eta), dev(g), gk, gv, gA, pos0, pos=pos)
    torch.cuda.synchronize()
    err = errors(y=(host(y), yo), A=(host(gA), oA), lse=(host(lse), lo[:, :, sl]))
    say("late position", err)
    for name, e in err.items():
        assert e <= bar(name, dtype), (name, e)
    assert np.array_equal(host(gk), okr) and np.array_equal(host(gv), ovr)
    assert np.all(pos.cpu().numpy() == pos0 + T1)
