"""C-ABI contract on the CPU: the library loads without a GPU, exports every
symbol include/tc.h declares, and rejects bad arguments on the host before
any HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import eviction_fed_weight_amd as tc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tc_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"tc_forward", "tc_decode_step", "tc_backward", "tc_forward_workspace_size",
            "tc_backward_workspace_size", "tc_status_string", "tc_version"} <= set(names)
    L = tc.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(6):
        assert tc.tc_status_string(s) != "unknown status"
    assert tc.tc_status_string(99) == "unknown status"


def fwd(shape, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, lam=FAKE + 0x300000,
                eta=FAKE + 0x300100, gate=FAKE + 0x300200, y=FAKE + 0x400000, A=None, lse=None,
                ws=None, wsb=0)
    args.update(kw)
    return tc.lib().tc_forward(ctypes.byref(shape), args["q"], args["k"], args["v"], args["lam"],
                               args["eta"], args["gate"], args["y"], args["A"], args["lse"],
                               args["ws"], args["wsb"], None)


def test_forward_delta_validation():
    """tc_forward_delta rejects what tc_forward rejects, and always needs
    its own workspace (which grows with the chunks of 64 evictions)."""
    L = tc.lib()

    def call(shape, **kw):
        args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, lam=FAKE + 0x300000, eta=FAKE + 0x300100,
                    gate=FAKE + 0x300200, y=FAKE + 0x400000, A=None, lse=None, ws=None, wsb=0)
        args.update(kw)
        return L.tc_forward_delta(ctypes.byref(shape), args["q"], args["k"], args["v"], args["lam"], args["eta"],
                                  args["gate"], args["y"], args["A"], args["lse"], args["ws"], args["wsb"], None)

    ok = tc.make_shape(1, 1, 64, 64, 8, 8)
    need = tc.tc_forward_delta_workspace_size(ok)
    assert need > 0 and need % 256 == 0
    assert tc.tc_forward_delta_workspace_size(tc.make_shape(1, 1, 64, 48, 8, 8)) == 0
    assert call(tc.make_shape(1, 1, 64, 48, 8, 8)) == tc.TC_ERR_UNSUPPORTED
    assert call(tc.make_shape(0, 1, 64, 64, 8, 8)) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(ok, q=None) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(ok, y=FAKE) == tc.TC_ERR_INVALID_ARGUMENT  # output aliasing an input
    assert call(ok) == tc.TC_ERR_WORKSPACE
    assert call(ok, ws=FAKE + 0x1000000, wsb=need - 1) == tc.TC_ERR_WORKSPACE
    assert call(ok, ws=FAKE + 0x3f0000, wsb=need) == tc.TC_ERR_INVALID_ARGUMENT  # ws overlaps y
    assert L.tc_forward_delta(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0,
                              None) == tc.TC_ERR_INVALID_ARGUMENT
    # more evictions, more chunks: a larger workspace
    assert tc.tc_forward_delta_workspace_size(tc.make_shape(1, 1, 64 * 40, 64, 8, 8)) > need


def test_forward_validation():
    ok = tc.make_shape(1, 1, 64, 64, 8, 8)
    assert fwd(tc.make_shape(1, 1, 64, 48, 8, 8)) == tc.TC_ERR_UNSUPPORTED
    assert fwd(tc.make_shape(1, 1, 64, 64, 8, 8, dtype=7)) == tc.TC_ERR_UNSUPPORTED
    for bad in [tc.make_shape(0, 1, 64, 64, 8, 8), tc.make_shape(1, 1, 0, 64, 8, 8),
                tc.make_shape(1, 1, 64, 64, 0, 8), tc.make_shape(1, 1, 64, 64, 8, 0),
                tc.make_shape(1, 0, 64, 64, 8, 8)]:
        assert fwd(bad) == tc.TC_ERR_INVALID_ARGUMENT
    assert fwd(ok, q=None) == tc.TC_ERR_INVALID_ARGUMENT
    assert fwd(ok, y=None) == tc.TC_ERR_INVALID_ARGUMENT
    assert fwd(ok, gate=None) == tc.TC_ERR_INVALID_ARGUMENT
    # output aliasing an input
    assert fwd(ok, y=FAKE) == tc.TC_ERR_INVALID_ARGUMENT
    assert fwd(ok, lse=FAKE + 0x100010) == tc.TC_ERR_INVALID_ARGUMENT
    assert tc.lib().tc_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0,
                               None) == tc.TC_ERR_INVALID_ARGUMENT
    # multi-segment shape without a workspace
    big = tc.make_shape(4, 16, 8192, 128, 512, 64)
    need = tc.tc_forward_workspace_size(big)
    assert need > 0
    G = 1 << 32  # spacing so the fake buffers do not overlap
    far = dict(q=G, k=2 * G, v=3 * G, lam=4 * G, eta=4 * G + 256, gate=4 * G + 512, y=5 * G)
    assert fwd(big, **far) == tc.TC_ERR_WORKSPACE
    assert fwd(big, ws=6 * G, wsb=need - 1, **far) == tc.TC_ERR_WORKSPACE
    assert fwd(big, ws=5 * G + 4096, wsb=need, **far) == tc.TC_ERR_INVALID_ARGUMENT  # ws overlaps y


def test_workspace_sizes():
    assert tc.tc_forward_workspace_size(tc.make_shape(1, 1, 64, 48, 8, 8)) == 0
    s2 = tc.make_shape(8, 8, 1024, 64, 256, 64)
    assert tc.tc_forward_workspace_size(s2) % 256 == 0
    assert tc.tc_forward_workspace_size(s2) >= 64 * 64 * 4


def test_forward_workspace_layout():
    """The forward workspace holds nseg + 1 float32 D x D state slots per (b,h)
    (segment states, and the last segment's local state) followed by one
    64-bit flag per segment and one 64-bit status word per workgroup (one
    workgroup per segment), each part rounded up to 256 bytes.  B=8 H=8
    T=1024 D=64 runs as eight one-block (128-row) segments per head."""
    BH, nseg, D = 64, 8, 64
    states = BH * (nseg + 1) * D * D * 4
    flags = -(-BH * nseg * 8 // 256) * 256
    assert tc.tc_forward_workspace_size(tc.make_shape(8, 8, 1024, 64, 256, 64)) == states + 2 * flags


def test_forward_status_validation():
    """tc_forward_status checks its arguments on the host first: a shape that
    needs no workspace (one segment) reports TC_OK without one; a shape that
    needs one reports a missing or short workspace; bad shapes and pos0 are
    rejected.  (None of these touches a device.)"""
    L = tc.lib()
    one = tc.make_shape(1, 1, 100, 64, 32, 64)
    assert tc.tc_forward_workspace_size(one) > 0
    assert L.tc_forward_status(ctypes.byref(one), 0, None, 0, None) == tc.TC_OK
    big = tc.make_shape(8, 8, 1024, 64, 256, 64)
    need = tc.tc_forward_workspace_size(big)
    assert L.tc_forward_status(ctypes.byref(big), 0, None, 0, None) == tc.TC_ERR_WORKSPACE
    assert L.tc_forward_status(ctypes.byref(big), 0, FAKE, need - 1, None) == tc.TC_ERR_WORKSPACE
    assert L.tc_forward_status(ctypes.byref(big), -1, FAKE, need, None) == tc.TC_ERR_INVALID_ARGUMENT
    assert L.tc_forward_status(ctypes.byref(tc.make_shape(1, 1, 64, 48, 8, 8)), 0, FAKE, need, None) \
        == tc.TC_ERR_UNSUPPORTED
    assert L.tc_forward_status(None, 0, FAKE, need, None) == tc.TC_ERR_INVALID_ARGUMENT


def test_continue_workspace_layout():
    """The continuation workspace is a forward workspace for the extended
    shape (p = min(pos0, W) ring rows + T new rows; whole blocks inside the
    prefix are not planned, so it is at most tc_forward's for that shape),
    then the float32 initial-state read [B,H,T,D] and the float32 state of
    this call's evictions [B,H,D,D], each part rounded up to 256 bytes (the
    forward reads the ring and the new tokens in place: no copy of the
    extended sequence)."""
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    for (B, H, T, D, W, pos0, es, dt) in [(2, 4, 512, 64, 256, 1000, 2, tc.TC_BF16), (1, 3, 100, 16, 8, 5, 4, tc.TC_F32),
                                          (1, 2, 300, 128, 128, 0, 2, tc.TC_BF16)]:
        p = min(pos0, W)
        tail = up(B * H * T * D * 4) + up(B * H * D * D * 4)
        fwd = tc.tc_continue_workspace_size(tc.make_shape(B, H, T, D, W, 64, 0.0, dt), pos0) - tail
        assert fwd > 0 and fwd % 256 == 0
        assert fwd <= tc.tc_forward_workspace_size(tc.make_shape(B, H, T + p, D, W, 64, 0.0, dt))
        if p == 0:  # nothing skipped: exactly the forward's workspace
            assert fwd == tc.tc_forward_workspace_size(tc.make_shape(B, H, T, D, W, 64, 0.0, dt))


def test_decode_validation():
    L = tc.lib()

    def call(shape, **kw):
        p = dict(q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, kr=FAKE + 0x100000, vr=FAKE + 0x200000,
                 A=FAKE + 0x300000, pos=FAKE + 0x400000, lam=FAKE + 0x500000, eta=FAKE + 0x500100,
                 gate=FAKE + 0x500200, y=FAKE + 0x600000)
        p.update(kw)
        return L.tc_decode_step(ctypes.byref(shape), p["q"], p["k"], p["v"], p["kr"], p["vr"],
                                p["A"], p["pos"], p["lam"], p["eta"], p["gate"], p["y"], None)

    assert call(tc.DecodeShape(1, 1, 48, 8, 0.0, 1)) == tc.TC_ERR_UNSUPPORTED
    assert call(tc.DecodeShape(0, 1, 64, 8, 0.0, 1)) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(tc.DecodeShape(1, 1, 64, 0, 0.0, 1)) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(tc.DecodeShape(1, 1, 64, 8, 0.0, 1), pos=None) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(tc.DecodeShape(1, 1, 64, 8, 0.0, 1), y=FAKE) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(tc.DecodeShape(1, 1, 64, 8, 0.0, 1), A=FAKE + 0x100000 + 64) == tc.TC_ERR_INVALID_ARGUMENT


def test_continue_validation():
    L = tc.lib()
    G = 1 << 32  # spacing so the fake buffers do not overlap

    def call(shape, pos0=300, **kw):
        p = dict(q=G, k=2 * G, v=3 * G, lam=4 * G, eta=4 * G + 256, gate=4 * G + 512, kr=5 * G, vr=6 * G,
                 A=7 * G, pos=8 * G, y=9 * G, lse=10 * G, ws=11 * G,
                 wsb=tc.tc_continue_workspace_size(shape, pos0))
        p.update(kw)
        return L.tc_forward_continue(ctypes.byref(shape), pos0, p["q"], p["k"], p["v"], p["lam"], p["eta"],
                                     p["gate"], p["kr"], p["vr"], p["A"], p["pos"], p["y"], p["lse"], p["ws"],
                                     p["wsb"], None)

    s = tc.make_shape(2, 4, 512, 64, 256, 64)
    assert tc.tc_continue_workspace_size(s, -1) == 0
    assert tc.tc_continue_workspace_size(tc.make_shape(1, 1, 64, 48, 8, 8), 0) == 0
    # the workspace depends on pos0 only through the ring prefix min(pos0, W) that joins the new tokens
    assert all(tc.tc_continue_workspace_size(s, p0) > 0 for p0 in (0, 100, 256))
    assert tc.tc_continue_workspace_size(s, 256) == tc.tc_continue_workspace_size(s, 10 ** 12)
    assert call(s, pos0=-1) == tc.TC_ERR_INVALID_ARGUMENT
    assert call(tc.make_shape(2, 4, 512, 48, 256, 64)) == tc.TC_ERR_UNSUPPORTED
    for name in ("q", "kr", "vr", "A", "y", "gate"):
        assert call(s, **{name: None}) == tc.TC_ERR_INVALID_ARGUMENT, name
    assert call(s, ws=None) == tc.TC_ERR_WORKSPACE
    assert call(s, wsb=tc.tc_continue_workspace_size(s, 300) - 1) == tc.TC_ERR_WORKSPACE
    assert call(s, y=G + 8) == tc.TC_ERR_INVALID_ARGUMENT           # misaligned
    assert call(s, kr=2 * G) == tc.TC_ERR_INVALID_ARGUMENT          # ring aliases the input keys
    assert call(s, A=6 * G + 4096) == tc.TC_ERR_INVALID_ARGUMENT    # memory inside the value ring
    assert call(s, ws=9 * G + 256) == tc.TC_ERR_INVALID_ARGUMENT    # workspace overlaps y
    assert call(s, pos=10 * G) == tc.TC_ERR_INVALID_ARGUMENT        # pos inside lse


def test_backward_validation():
    L = tc.lib()
    s = tc.make_shape(1, 1, 64, 48, 8, 8)
    args = [FAKE + i * 0x100000 for i in range(15)]
    assert L.tc_backward(ctypes.byref(s), *args, None, 0, None) == tc.TC_ERR_UNSUPPORTED
    s = tc.make_shape(1, 1, 64, 64, 8, 8)
    args2 = list(args)
    args2[0] = None
    assert L.tc_backward(ctypes.byref(s), *args2, None, 0, None) == tc.TC_ERR_INVALID_ARGUMENT


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 16)
    with pytest.raises(ValueError):
        tc.tc_forward(q, q, q, torch.zeros(1), torch.zeros(1), torch.zeros(1), 4)


def test_binding_checks_layouts_before_the_library():
    """The binding compares every tensor with the layout include/tc.h
    documents for it (the C ABI only sees pointers, so a short output or a
    wrong element type would be written out of bounds): wrong shapes, dtypes
    and lengths raise ValueError naming the tensor, before any device check."""
    torch = pytest.importorskip("torch")
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(1, 2, 8, 16, dtype=bf)
    p = torch.zeros(2)

    def raises(fn, name):
        with pytest.raises(ValueError) as e:
            fn()
        assert str(e.value).startswith(name), (name, str(e.value))

    # forward: short y, bf16 A_final, lse of the wrong length, lam of the wrong length or dtype, k of another dtype
    raises(lambda: tc.tc_forward(q, q, q, p, p, p, 4, y=torch.zeros(1, 2, 7, 16, dtype=bf)), "y")
    raises(lambda: tc.tc_forward(q, q, q, p, p, p, 4, A_final=torch.zeros(1, 2, 16, 16, dtype=bf)), "A_final")
    raises(lambda: tc.tc_forward(q, q, q, p, p, p, 4, lse=torch.zeros(1, 2, 9)), "lse")
    raises(lambda: tc.tc_forward(q, q, q, torch.zeros(3), p, p, 4), "lam")
    raises(lambda: tc.tc_forward(q, q, q, p, p, torch.zeros(2, dtype=torch.float64), 4), "gate")
    raises(lambda: tc.tc_forward(q, q.float(), q, p, p, p, 4), "k")
    # decode: int32 pos, bf16 A, ring of another width than q
    S, H, W, D = 2, 2, 8, 16
    qd = torch.zeros(S, H, D, dtype=bf)
    ring = torch.zeros(S, H, W, D, dtype=bf)
    A = torch.zeros(S, H, D, D)
    pos = torch.zeros(S, dtype=torch.int64)
    raises(lambda: tc.tc_decode_step(qd, qd, qd, ring, ring, A, pos.int(), p, p, p), "pos")
    raises(lambda: tc.tc_decode_step(qd, qd, qd, ring, ring, A.to(bf), pos, p, p, p), "A")
    raises(lambda: tc.tc_decode_step(qd, qd, qd, ring, torch.zeros(S, H, W, 32, dtype=bf), A, pos, p, p, p),
           "v_ring")
    raises(lambda: tc.tc_decode_step(qd, qd, qd, ring, ring, A, pos, p, p, p, y=torch.zeros(S, H, D, dtype=f32)),
           "y")
    # continuation: memory of another batch, pos as int32
    raises(lambda: tc.tc_forward_continue(q, q, q, p, p, p, torch.zeros(1, 2, W, 16, dtype=bf),
                                          torch.zeros(1, 2, W, 16, dtype=bf), torch.zeros(2, 2, 16, 16), 0), "A")
    raises(lambda: tc.tc_forward_continue(q, q, q, p, p, p, torch.zeros(1, 2, W, 16, dtype=bf),
                                          torch.zeros(1, 2, W, 16, dtype=bf), torch.zeros(1, 2, 16, 16), 0,
                                          pos=torch.zeros(1, dtype=torch.int32)), "pos")
    # backward: lse of the wrong dtype, short dq
    lse = torch.zeros(1, 2, 8)
    raises(lambda: tc.tc_backward(q, q, q, q, q, lse.double(), p, p, p, 4), "lse")
    raises(lambda: tc.tc_backward(q, q, q, q, q, lse, p, p, p, 4, dq=torch.zeros(1, 2, 8, 8, dtype=bf)), "dq")
