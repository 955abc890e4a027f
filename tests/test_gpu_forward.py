"""GPU parity of tc_forward (through the C ABI) against the CPU oracle."""
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


def run_and_compare(d, W, C=64, heads=None, check_state=True, status=False):
    """Run the GPU forward on all of d, compare (optionally a subset of heads
    (b, h) list) against the oracle.  Returns the error dict.  status: also
    check that tc_forward_status reports the call complete."""
    dtype = d["dtype"]
    q, k, v = (dev(d[x], dtype) for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    m = tc()
    shape = m.make_shape(*q.shape, W, C, 0.0, m.TC_BF16 if dtype == "bf16" else m.TC_F32)
    ws = torch.empty(max(m.tc_forward_workspace_size(shape), 1), dtype=torch.uint8, device="cuda")
    y, A, lse = m.tc_forward(q, k, v, lam, eta, g, W, C, ws=ws)
    if status:
        assert m.tc_forward_status(shape, ws) == m.TC_OK
    torch.cuda.synchronize()
    y, A, lse = host(y), host(A), host(lse)
    if heads is None:
        yo, Ao, lo = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], W)
        err = errors(y=(y, yo), A=(A, Ao), lse=(lse, lo))
    else:
        err = {}
        for b, h in heads:
            sl = lambda x: x[b:b + 1, h:h + 1]  # noqa: E731
            yo, Ao, lo = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["lam"][h:h + 1],
                                        d["eta"][h:h + 1], d["gate"][h:h + 1], W)
            for key, e in errors(y=(sl(y), yo), A=(sl(A), Ao), lse=(sl(lse), lo)).items():
                err[key] = max(err.get(key, 0.0), e)
    if not check_state:
        err.pop("A")
        err.pop("A_row")
    return err


SMALL = [
    # B, H, T, D, W, dtype
    (1, 1, 64, 16, 8, "f32"),
    (2, 3, 200, 16, 8, "f32"),
    (1, 2, 333, 32, 64, "f32"),
    (2, 2, 300, 64, 100, "f32"),
    (1, 2, 257, 128, 64, "f32"),
    (2, 3, 200, 16, 8, "bf16"),
    (1, 2, 333, 32, 64, "bf16"),
    (2, 2, 500, 64, 100, "bf16"),
    (2, 2, 512, 64, 256, "bf16"),
    (1, 2, 449, 128, 128, "bf16"),
    (1, 1, 1, 64, 1, "bf16"),
    (1, 1, 5, 16, 1, "f32"),
    (1, 2, 100, 64, 1, "bf16"),
    (1, 2, 130, 64, 200, "bf16"),   # W > T: pure causal softmax, A = 0
    (1, 1, 64, 64, 64, "bf16"),     # W = T
    (1, 2, 65, 16, 64, "f32"),      # one eviction
]


@pytest.mark.parametrize("B,H,T,D,W,dtype", SMALL)
def test_forward_small(B, H, T, D, W, dtype):
    say("forward", B, H, T, D, W, dtype)
    d = tc_inputs.prefill_inputs(2, seed=17 + T + D, B=B, H=H, T=T, D=D, W=W, dtype=dtype, plants=False)
    err = run_and_compare(d, W)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, dtype), (key, e)


@pytest.mark.parametrize("lam,eta,gate", [(0.0, 0.5, 0.3), (1.0, 0.25, -0.5), (0.9, 0.0, 0.0),
                                          (0.95, 0.7, -60.0), (0.5, 2.0, 3.0)])
def test_forward_parameter_edges(lam, eta, gate):
    say("forward edges", lam, eta, gate)
    d = tc_inputs.prefill_inputs(2, seed=5, B=1, H=2, T=300, D=64, W=70, dtype="f32", plants=False)
    d["lam"][:] = lam
    d["eta"][:] = eta
    d["gate"][:] = gate
    err = run_and_compare(d, 70)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "f32"), (key, e)


def test_forward_multi_segment_walk():
    """Enough blocks that workgroups walk several blocks and segment-start
    states come from the per-segment pass and the chain."""
    say("forward multi-segment")
    d = tc_inputs.prefill_inputs(2, seed=3, B=1, H=2, T=64 * 520 + 17, D=16, W=100, dtype="f32",
                                 plants=False)
    err = run_and_compare(d, 100)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "f32"), (key, e)


def test_forward_multi_segment_walk_bf16():
    say("forward multi-segment bf16")
    d = tc_inputs.prefill_inputs(2, seed=4, B=2, H=4, T=64 * 140, D=64, W=320, dtype="bf16",
                                 plants=False)
    err = run_and_compare(d, 320, heads=[(0, 0), (1, 3)])
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


@pytest.mark.parametrize("T", [2048, 2048 + 50])
def test_forward_segment_prefix_paths(T):
    """bf16 D=64 with one block per segment: 16 segments (the fused kernel
    combines the local segment states itself) and 17 with a ragged last block
    (the chain kernel combines them)."""
    say("forward segment prefix", T)
    d = tc_inputs.prefill_inputs(2, seed=21, B=1, H=2, T=T, D=64, W=300, dtype="bf16", plants=False)
    err = run_and_compare(d, 300)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


@pytest.mark.parametrize("T", [1024, 1024 + 37])
def test_forward_blocks_per_segment_bf16(T):
    """Many heads, short sequences: each workgroup walks several 128-row
    blocks, carrying the state through its chunk updates; the final state
    comes from the last segment's local state (with a ragged last block for
    T = 1061)."""
    say("forward several blocks per segment", T)
    d = tc_inputs.prefill_inputs(2, seed=22, B=4, H=64, T=T, D=64, W=200, dtype="bf16", plants=False)
    err = run_and_compare(d, 200, heads=[(0, 0), (1, 33), (3, 63)])
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_forward_config1_tiny_fp32():
    d = tc_inputs.prefill_inputs(1)
    err = run_and_compare(d, 8, C=8)
    say("config 1", err)
    for key, e in err.items():
        assert e <= bar(key, "f32"), (key, e)


def test_forward_config2_full():
    d = tc_inputs.prefill_inputs(2)
    err = run_and_compare(d, 256, C=64)
    say("config 2", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_forward_config3_sampled_heads():
    """Full 32,768-token, 12-head launch; the oracle checks two whole heads."""
    d = tc_inputs.prefill_inputs(3)
    err = run_and_compare(d, 1024, C=128, heads=[(0, 0), (0, 7)])
    say("config 3", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_forward_config5_sampled_heads():
    d = tc_inputs.prefill_inputs(5, with_dy=False)
    err = run_and_compare(d, 512, C=64, heads=[(0, 0), (3, 15)])
    say("config 5 forward", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_forward_deterministic():
    d = tc_inputs.prefill_inputs(2, seed=9, B=2, H=4, T=640, D=64, W=192, plants=False)
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    outs = [tc().tc_forward(q, k, v, lam, eta, g, 192) for _ in range(3)]
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a, b)


@pytest.mark.parametrize("D", [16, 32, 64])
def test_forward_state_exchange(D):
    """One block per segment: each workgroup publishes the local state of its
    evicted chunk and later segments of the head sum the published states."""
    say("forward state exchange", D)
    d = tc_inputs.prefill_inputs(2, seed=31 + D, B=2, H=4, T=1024 + 37, D=D, W=200, dtype="bf16", plants=False)
    err = run_and_compare(d, 200, status=True)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


def test_forward_flag_wait_runs_out(monkeypatch):
    """TC_FORWARD_MAX_POLLS=0 ends every flag wait at once: the kernel still
    finishes, the blocks that needed earlier segments' states come back NaN
    (never a stale state), every other row matches the oracle, and
    tc_forward_status reports the call (TC_ERR_STATE_EXCHANGE).  A later call
    on the same workspace with the normal bound reports TC_OK."""
    say("forward flag wait runs out")
    m = tc()
    monkeypatch.setenv("TC_FORWARD_MAX_POLLS", "0")
    B, H, D, W, T = 2, 4, 64, 200, 1024 + 37
    d = tc_inputs.prefill_inputs(2, seed=33, B=B, H=H, T=T, D=D, W=W, dtype="bf16", plants=False)
    q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
    shape = m.make_shape(B, H, T, D, W, 64, 0.0, m.TC_BF16)
    ws = torch.empty(m.tc_forward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    y, A, _ = m.tc_forward(q, k, v, lam, eta, g, W, ws=ws)
    assert m.tc_forward_status(shape, ws) == m.TC_ERR_STATE_EXCHANGE
    y, A = host(y), host(A)
    cut = (W // 128 + 1) * 128  # first row of the first block that sums earlier segments' states
    assert np.isnan(y[:, :, cut:]).all() and np.isnan(A).all()
    yo, Ao, _ = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], W)
    err = errors(y=(y[:, :, :cut], yo[:, :, :cut]))
    say("  error of the other rows", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)
    monkeypatch.delenv("TC_FORWARD_MAX_POLLS")
    y2, A2, _ = m.tc_forward(q, k, v, lam, eta, g, W, ws=ws)
    assert m.tc_forward_status(shape, ws) == m.TC_OK
    err = errors(y=(host(y2), yo), A=(host(A2), Ao))
    say("  the next call", err)
    for key, e in err.items():
        assert e <= bar(key, "bf16"), (key, e)


@pytest.mark.parametrize("B,H,T,D,W", [(2, 4, 4096 + 37, 128, 200), (1, 3, 64 * 70 + 23, 128, 128)])
def test_forward_f32_d128_multi_segment(B, H, T, D, W):
    """float32 with D = 128 (state in LDS, matrix-core results in VGPRs),
    T > 4096 with a ragged last block, several 64-row blocks per workgroup
    segment (B*H*blocks > 256) and segment-start states from the state pass
    and the chain; W not a multiple of the block and W = 128."""
    say("forward f32 D=128 multi-segment", B, H, T, D, W)
    d = tc_inputs.prefill_inputs(2, seed=61 + W, B=B, H=H, T=T, D=D, W=W, dtype="f32", plants=False)
    err = run_and_compare(d, W)
    say("  errors", err)
    for key, e in err.items():
        assert e <= bar(key, "f32"), (key, e)


def test_forward_workspace_reuse():
    """One workspace filled with arbitrary bytes, then reused by calls on
    different inputs: flags left by a call (or by the initial contents) must
    never be taken for those of a later call."""
    say("forward workspace reuse")
    T, W = 1024, 256
    d1 = tc_inputs.prefill_inputs(2, seed=41, B=2, H=4, T=T, D=64, W=W, dtype="bf16", plants=False)
    d2 = tc_inputs.prefill_inputs(2, seed=42, B=2, H=4, T=T, D=64, W=W, dtype="bf16", plants=False)
    m = tc()
    nbytes = m.tc_forward_workspace_size(m.make_shape(2, 4, T, 64, W, 64, 0.0, m.TC_BF16))
    gen = torch.Generator().manual_seed(7)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen).to("cuda")
    ref = {}
    for i, d in enumerate((d1, d2, d1, d2)):
        q, k, v = (dev(d[x], "bf16") for x in ("q", "k", "v"))
        lam, eta, g = (dev(d[x], "f32") for x in ("lam", "eta", "gate"))
        y, A, lse = m.tc_forward(q, k, v, lam, eta, g, W, ws=ws)
        torch.cuda.synchronize()
        y, A = host(y), host(A)
        if i < 2:
            yo, Ao, _ = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], W)
            err = errors(y=(y, yo), A=(A, Ao))
            say("  call", i, "errors", err)
            for key, e in err.items():
                assert e <= bar(key, "bf16"), (i, key, e)
            ref[i] = (y, A)
        else:
            assert np.array_equal(y, ref[i - 2][0]) and np.array_equal(A, ref[i - 2][1]), i


def test_forward_graph_capture():
    """tc_forward captured in a HIP graph and replayed on new inputs, with
    eager calls between the replays: every replay and every eager call
    matches the oracle.  (Under capture the launcher takes the path without
    inter-workgroup flags: a replay repeats the captured flag value.)"""
    say("forward graph capture")
    B, H, T, D, W = 2, 4, 1024, 64, 256
    ds = [tc_inputs.prefill_inputs(2, seed=51 + i, B=B, H=H, T=T, D=D, W=W, dtype="bf16", plants=False)
          for i in range(3)]
    m = tc()
    q, k, v = (dev(ds[0][x], "bf16") for x in ("q", "k", "v"))
    lam, eta, g = (dev(ds[0][x], "f32") for x in ("lam", "eta", "gate"))
    ws = torch.empty(m.tc_forward_workspace_size(m.make_shape(B, H, T, D, W, 64, 0.0, m.TC_BF16)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(q)
    A = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.tc_forward(q, k, v, lam, eta, g, W, y=y, A_final=A, lse=lse, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.tc_forward(q, k, v, lam, eta, g, W, y=y, A_final=A, lse=lse, ws=ws)
    torch.cuda.synchronize()
    for i in (1, 2, 0, 1):
        d = ds[i]
        for dst, x in ((q, "q"), (k, "k"), (v, "v")):
            dst.copy_(dev(d[x], "bf16"))
        for dst, x in ((lam, "lam"), (eta, "eta"), (g, "gate")):
            dst.copy_(dev(d[x], "f32"))
        graph.replay()
        torch.cuda.synchronize()
        yo, Ao, lo = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], W)
        err = errors(y=(host(y), yo), A=(host(A), Ao), lse=(host(lse), lo))
        say("  replay on inputs", i, err)
        for key, e in err.items():
            assert e <= bar(key, "bf16"), ("replay", i, key, e)
        ye, Ae, _ = m.tc_forward(q, k, v, lam, eta, g, W, ws=ws)  # eager call on the same workspace
        torch.cuda.synchronize()
        ee = errors(y=(host(ye), yo), A=(host(Ae), Ao))
        for key, e in ee.items():
            assert e <= bar(key, "bf16"), ("eager", i, key, e)


def test_forward_concurrent_streams():
    """Two forwards of the state-exchange shape on two streams at once (each
    with its own workspace), several times over: both match the oracle.  The
    other stream's kernel holds compute units, so the grid need not be
    resident; a workgroup waits only for earlier-dispatched workgroups of its
    own launch, so every wait still ends."""
    B, H, T, D, W = 8, 8, 1024, 64, 256
    m = tc()
    ds = [tc_inputs.prefill_inputs(2, seed=71 + i, B=B, H=H, T=T, D=D, W=W, dtype="bf16", plants=False)
          for i in range(2)]
    ins = [[dev(d[x], "bf16") for x in ("q", "k", "v")] + [dev(d[x], "f32") for x in ("lam", "eta", "gate")]
           for d in ds]
    shape = m.make_shape(B, H, T, D, W, 64, 0.0, m.TC_BF16)
    wss = [torch.empty(m.tc_forward_workspace_size(shape), dtype=torch.uint8, device="cuda") for _ in ds]
    outs = [[torch.empty_like(x[0]), torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")] for x in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(5):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                m.tc_forward(*ins[i], W, y=outs[i][0], A_final=outs[i][1], want_lse=False, ws=wss[i])
        torch.cuda.synchronize()
    for i, d in enumerate(ds):
        yo, Ao, _ = oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], W)
        err = errors(y=(host(outs[i][0]), yo), A=(host(outs[i][1]), Ao))
        say("  stream", i, err)
        for key, e in err.items():
            assert e <= bar(key, "bf16"), (i, key, e)
