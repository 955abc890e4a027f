"""Benchmark of the TC layer hot path on one MI355X.

Headline (the JSON line's "value"): prefill tokens/s of tc_forward on the
long-context workload B=1 H=12 D=64 T=32768 W=1024 C=128 bf16 (the largest
prefill that one GPU holds; B*T tokens per call, inputs resident in HBM).
The same line carries the training-shape prefill (B=8 H=8 T=1024), the
decode rate of the serving workload (64 streams x 32 heads, D=128, W=4096:
tc_decode_step calls per second), the backward and the training-shape
forward, each with its roofline, plus the CPU oracle timed on the host on
bounded samples of the same workloads.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
                    [--legs prefill,decode,backward,train_forward,continue,chunk_mean,capacity[,calib]]

The long-context prefill (the headline) always runs; --legs picks the others.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0  # TFLOP/s, MI355X dense bf16 MFMA
PEAK_HBM = 8000.0   # GB/s, MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "eviction_fed_weight_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_pmc.txt")


def csrc_digest():
    """sha256 over the library's HIP sources (names and bytes, sorted)."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per call of each leg from the committed profiler summary
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a copy of known size), or {}
    when the kernels changed after the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return {}
    kv = {}
    for ln in lines:
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("csrc_sha256") != csrc_digest():
        return {}
    out = {}
    for leg in ("prefill", "long", "decode", "backward", "train_forward", "continue"):
        key = "%s_bytes_per_call" % leg
        if key in kv:
            out[leg] = float(kv[key])
    return out


def kernel_chunk(D, dtype="bf16"):
    """Evictions per read chunk of the forward kernels: a query block of 128
    rows (bf16) or 64 rows (float32) reads q S(e0) for the state before the
    block's evicted chunk plus the decayed triangle over that chunk, so the
    kernel's intra-chunk term is that of C = 128 or 64."""
    return 128 if dtype == "bf16" else 64


def roofline_chunk(C, D, dtype="bf16"):
    """The chunk the algorithmic flops are charged with: the workload's C,
    but never more than the kernel's read chunk (a larger C would charge
    intra-chunk work the kernel does not do)."""
    return min(C, kernel_chunk(D, dtype))


def fwd_flops(B, H, T, D, W, C):
    """Algorithmic forward FLOPs: band QK^T+PV (4D per pair) plus the memory
    write (2D^2), read (2D^2) and intra-chunk triangle (2D(C+1)) per evicted
    query."""
    P = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
    E = max(T - W, 0)
    return B * H * (4 * D * P + E * (4 * D * D + 2 * D * (C + 1)))


def fwd_bytes(B, H, T, D, e_in=2, e_out=2):
    return B * H * (T * D * (3 * e_in + e_out) + 4 * D * D + 4 * T)


def bwd_flops(B, H, T, D, W, C):
    P = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
    E = max(T - W, 0)
    return B * H * (10 * D * P + E * (10 * D * D + 4 * D * (C + 1)))


def decode_bytes(S, H, D, W, e=2):
    return S * H * (2 * W * D * e + 2 * D * e + 8 * D * D + 4 * D * e)


def time_calls(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def cold_ms(fn, n, flush_mib=512):
    """Median time of n single calls, each after a 512 MiB device write so
    that no input is left in the 256 MB Infinity Cache (inputs in HBM)."""
    import torch

    buf = torch.empty(flush_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    times = []
    for i in range(n):
        buf.fill_(float(i))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    del buf
    return times[len(times) // 2]


def prefill_leg(cfg_id, steps, warmup):
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    cfg = tc_inputs.CONFIGS[cfg_id]
    d = tc_inputs.prefill_inputs(cfg_id, with_dy=False) if cfg_id == 5 else tc_inputs.prefill_inputs(cfg_id)
    dv = torch.device("cuda")
    q, k, v = (torch.from_numpy(d[x]).to(dv).to(torch.bfloat16).contiguous() for x in ("q", "k", "v"))
    lam, eta, g = (torch.from_numpy(d[x]).to(dv) for x in ("lam", "eta", "gate"))
    y = torch.empty_like(q)
    A = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dv)
    lse = torch.empty((cfg.B, cfg.H, cfg.T), dtype=torch.float32, device=dv)
    shape = tc.make_shape(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, cfg.C)
    ws = torch.empty(max(tc.tc_forward_workspace_size(shape), 1), dtype=torch.uint8, device=dv)

    def call():
        tc.tc_forward(q, k, v, lam, eta, g, cfg.W, cfg.C, y=y, A_final=A, lse=lse, ws=ws)

    ms = time_calls(call, steps, warmup)
    fl = fwd_flops(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, roofline_chunk(cfg.C, cfg.D))
    by = fwd_bytes(cfg.B, cfg.H, cfg.T, cfg.D)
    tflops = fl / (ms * 1e-3) / 1e12
    cold = cold_ms(call, 20) if cfg_id in (2, 3) else None
    return dict(
        workload="%s B=%d H=%d D=%d T=%d W=%d C=%d bf16" % ("forward" if cfg_id == 5 else "prefill", cfg.B, cfg.H, cfg.D,
                                                           cfg.T, cfg.W, cfg.C),
        ms_per_call=ms, tokens_per_s=cfg.B * cfg.T / (ms * 1e-3), flops=fl, bytes=by,
        roofline=dict(bound="mfma", achieved=tflops, peak=PEAK_BF16, unit="TFLOP/s", frac=tflops / PEAK_BF16,
                      traffic=measured_traffic().get({2: "prefill", 3: "long", 5: "train_forward"}[cfg_id]),
                      kernel=("one tc_forward call (fwd_kernel_rows; with several blocks per segment also "
                              "seg_state_kernel [+ seg_chain_kernel])" if cfg.D <= 64 else
                              "one tc_forward call (seg_state_kernel in parts + seg_chain_kernel + fwd_kernel, "
                              "D=128: 128-row blocks on eight waves, state in LDS)")),
        hbm_gbs=by / (ms * 1e-3) / 1e9,
        cold=None if cold is None else dict(
            ms_per_call=cold, tokens_per_s=cfg.B * cfg.T / (cold * 1e-3), tflops=fl / (cold * 1e-3) / 1e12,
            frac=fl / (cold * 1e-3) / 1e12 / PEAK_BF16,
            note="median of 20 single calls, each after writing 512 MiB (the 256 MB Infinity Cache holds no input)"),
    )


def continue_leg(steps, warmup, chunk=4096):
    """Chunked prefill of the long-context workload (B=1 H=12 D=64 T=32768
    W=1024): the sequence in chunks of `chunk` tokens, each a
    tc_forward_continue call from the ring and memory the previous one left.
    One step = the whole sequence (T / chunk calls), timed from an empty state
    each time."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    cfg = tc_inputs.CONFIGS[3]
    d = tc_inputs.prefill_inputs(3)
    dv = torch.device("cuda")
    q, k, v = (torch.from_numpy(d[x]).to(dv).to(torch.bfloat16).contiguous() for x in ("q", "k", "v"))
    lam, eta, g = (torch.from_numpy(d[x]).to(dv) for x in ("lam", "eta", "gate"))
    B, H, T, D, W = cfg.B, cfg.H, cfg.T, cfg.D, cfg.W
    n = (T + chunk - 1) // chunk
    parts = [tuple(x[:, :, i * chunk:(i + 1) * chunk].contiguous() for x in (q, k, v)) for i in range(n)]
    ys = [torch.empty_like(p[0]) for p in parts]
    lses = [torch.empty((B, H, p[0].shape[2]), dtype=torch.float32, device=dv) for p in parts]
    kr = torch.zeros((B, H, W, D), dtype=torch.bfloat16, device=dv)
    vr = torch.zeros_like(kr)
    A = torch.zeros((B, H, D, D), dtype=torch.float32, device=dv)
    pos = torch.zeros(B, dtype=torch.int64, device=dv)
    shape = tc.make_shape(B, H, chunk, D, W, cfg.C)
    ws = torch.empty(tc.tc_continue_workspace_size(shape, W), dtype=torch.uint8, device=dv)

    def call():
        A.zero_()
        for i, (qi, ki, vi) in enumerate(parts):
            tc.tc_forward_continue(qi, ki, vi, lam, eta, g, kr, vr, A, i * chunk, pos=pos, C=cfg.C,
                                   y=ys[i], lse=lses[i], ws=ws)

    ms = time_calls(call, steps, warmup)
    fl = fwd_flops(B, H, T, D, W, roofline_chunk(cfg.C, D))
    tflops = fl / (ms * 1e-3) / 1e12
    return dict(workload="chunked prefill B=%d H=%d D=%d T=%d W=%d C=%d bf16 in %d chunks of %d"
                % (B, H, D, T, W, cfg.C, n, chunk),
                ms_per_sequence=ms, tokens_per_s=B * T / (ms * 1e-3), flops=fl,
                roofline=dict(bound="mfma", achieved=tflops, peak=PEAK_BF16, unit="TFLOP/s", frac=tflops / PEAK_BF16,
                              traffic=measured_traffic().get("continue"),
                              kernel="%d tc_forward_continue calls (each: the forward over the ring prefix and "
                                     "the chunk, its segments exchanging states seeded from the carried memory, "
                                     "then the ring and memory update)" % n))


def chunk_mean_leg(steps, warmup, exact_ms):
    """The chunk-mean shortcut (one mean write per chunk of C evicted pairs)
    on the long-context workload, next to the exact scan: its time per call,
    the cost ratio shortcut / exact, and how far its output lands from the
    exact one (relative L2 over y) -- the pages claim the exact scan comes at
    the same computational cost and removes the C^2 - C cross terms per chunk
    ("Tensor Cache: Eviction-conditioned Associative Memory for
    Transformers", abstract and Section 1)."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    cfg = tc_inputs.CONFIGS[3]
    d = tc_inputs.prefill_inputs(3)
    dv = torch.device("cuda")
    q, k, v = (torch.from_numpy(d[x]).to(dv).to(torch.bfloat16).contiguous() for x in ("q", "k", "v"))
    lam, eta, g = (torch.from_numpy(d[x]).to(dv) for x in ("lam", "eta", "gate"))
    y = torch.empty_like(q)
    A = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dv)
    lse = torch.empty((cfg.B, cfg.H, cfg.T), dtype=torch.float32, device=dv)
    shape = tc.make_shape(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, cfg.C)
    ws = torch.empty(max(tc.tc_forward_workspace_size(shape), 1), dtype=torch.uint8, device=dv)

    def call():
        tc.tc_forward_chunk_mean(q, k, v, lam, eta, g, cfg.W, cfg.C, y=y, A_final=A, lse=lse, ws=ws)

    ms = time_calls(call, steps, warmup)
    ye, Ae, _ = tc.tc_forward(q, k, v, lam, eta, g, cfg.W, cfg.C)
    torch.cuda.synchronize()
    gap = float((y.float() - ye.float()).norm() / ye.float().norm())
    gap_m = float((A - Ae).norm() / Ae.norm())
    return dict(workload="chunk-mean shortcut, prefill B=%d H=%d D=%d T=%d W=%d C=%d bf16" % (cfg.B, cfg.H, cfg.D, cfg.T,
                                                                                            cfg.W, cfg.C),
                ms_per_call=ms, tokens_per_s=cfg.B * cfg.T / (ms * 1e-3), exact_ms_per_call=exact_ms,
                cost_ratio_shortcut_over_exact=ms / exact_ms, rel_gap_y_vs_exact=gap, rel_gap_A_final_vs_exact=gap_m,
                kernel="one tc_forward_chunk_mean call (seg_state_kernel [mean writes] + seg_chain_kernel + "
                       "fwd_kernel_rows, no intra-chunk terms)")


def delta_leg(steps, warmup, exact_ms):
    """The delta-rule write variant (the optional write of Figure 2, step 3,
    of "Tensor Cache: Eviction-conditioned Associative Memory for
    Transformers"; reading: the evicted key's prediction error is written) on
    the long-context and the training-shape prefill: time per call, cost
    ratio over the outer-product layer (exact scan) and the relative distance
    of its output from it.  exact_ms: {cfg_id: ms per tc_forward call}."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    out = []
    for cfg_id in (3, 2):
        cfg = tc_inputs.CONFIGS[cfg_id]
        d = tc_inputs.prefill_inputs(cfg_id)
        dv = torch.device("cuda")
        q, k, v = (torch.from_numpy(d[x]).to(dv).to(torch.bfloat16).contiguous() for x in ("q", "k", "v"))
        lam, eta, g = (torch.from_numpy(d[x]).to(dv) for x in ("lam", "eta", "gate"))
        y = torch.empty_like(q)
        A = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dv)
        lse = torch.empty((cfg.B, cfg.H, cfg.T), dtype=torch.float32, device=dv)
        shape = tc.make_shape(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, cfg.C)
        ws = torch.empty(tc.tc_forward_delta_workspace_size(shape), dtype=torch.uint8, device=dv)

        def call():
            tc.tc_forward_delta(q, k, v, lam, eta, g, cfg.W, cfg.C, y=y, A_final=A, lse=lse, ws=ws)

        ms = time_calls(call, max(3, steps // 10), max(1, warmup // 10))
        ye, Ae, _ = tc.tc_forward(q, k, v, lam, eta, g, cfg.W, cfg.C)
        torch.cuda.synchronize()
        out.append(dict(
            workload="delta-rule write, prefill B=%d H=%d D=%d T=%d W=%d bf16" % (cfg.B, cfg.H, cfg.D, cfg.T, cfg.W),
            ms_per_call=ms, tokens_per_s=cfg.B * cfg.T / (ms * 1e-3), exact_ms_per_call=exact_ms.get(cfg_id),
            cost_ratio_delta_over_exact=(ms / exact_ms[cfg_id]) if cfg_id in exact_ms else None,
            rel_gap_y_vs_exact=float((y.float() - ye.float()).norm() / ye.float().norm()),
            rel_gap_A_final_vs_exact=float((A - Ae).norm() / Ae.norm()),
            kernel="one tc_forward_delta call (delta_chunk_kernel [per chunk of 64 evictions] + delta_group_kernel "
                   "[per level] + delta_walk_kernel [one workgroup per head] + delta_expand_kernel [upper levels] + "
                   "delta_expand_read_kernel [per group of chunks: the last expansion and the read] + the "
                   "window-only forward)"))
    return out


def capacity_leg(D=128, H=8, Ns=(64, 128, 256, 512, 1024, 2048, 4096)):
    """Raw memory-capacity diagnostic (the "memory-capacity diagnostics" of the
    abstract of "Tensor Cache: Eviction-conditioned Associative Memory for
    Transformers"; parameters are not given there): N unit-norm keys with N(0,1) values
    written into A (window 1, lambda = eta = 1), then read back with the
    stored keys; recall@1 = fraction of reads whose nearest stored value (by
    cosine) is their own.  One tc_forward call of 2N tokens per N."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    dv = torch.device("cuda")
    out = []
    for N in Ns:
        q, k, v, lam, eta, g, vals = tc_inputs.capacity_inputs(N, D, H)
        Q, K, V = (torch.from_numpy(x).to(dv).to(torch.bfloat16) for x in (q, k, v))
        L, E, G = (torch.from_numpy(x).to(dv) for x in (lam, eta, g))
        y, _, _ = tc.tc_forward(Q, K, V, L, E, G, 1, 64, want_state=False, want_lse=False)
        ms = time_calls(lambda: tc.tc_forward(Q, K, V, L, E, G, 1, 64, y=y, want_state=False, want_lse=False), 5, 2)
        r = torch.nn.functional.normalize(y[0, :, N:].float(), dim=-1)
        st = torch.nn.functional.normalize(torch.from_numpy(vals).to(dv).float(), dim=-1)
        hit = (torch.bmm(r, st.transpose(1, 2).contiguous()).argmax(-1) == torch.arange(N, device=dv)).float()
        out.append(dict(N=N, N_over_D=N / D, recall_at_1=hit.mean().item(), ms_per_call=ms))
    return dict(workload="capacity probe D=%d H=%d bf16: N pairs written, then read with their keys" % (D, H),
                points=out)


def decode_leg(steps, warmup):
    """Serving decode: 64 streams x 32 heads, D=128, W=4096.  The start state
    (ring of the last 4,096 pairs, A after 8,192 prior evictions) is built on
    the device from seeded draws, A with the library's own forward pass."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    cfg = tc_inputs.CONFIGS[4]
    S, H, D, W = cfg.S, cfg.H, cfg.D, cfg.W
    dv = torch.device("cuda")
    lam, eta, g = (torch.from_numpy(x).to(dv) for x in tc_inputs.decode_params(4, H))
    gen = torch.Generator(device=dv)
    gen.manual_seed(4)
    bf = torch.bfloat16
    # A after `prior` evictions = the state tc_forward reaches with W=1 over prior+1 tokens
    pk = torch.randn((S, H, cfg.prior + 1, D), generator=gen, device=dv).to(bf)
    pv = torch.randn((S, H, cfg.prior + 1, D), generator=gen, device=dv).to(bf)
    pq = torch.zeros_like(pk)
    _, A, _ = tc.tc_forward(pq.view(S, H, -1, D), pk, pv, lam, eta, g, 1, 64, want_lse=False)
    del pk, pv, pq
    kr = torch.randn((S, H, W, D), generator=gen, device=dv).to(bf)
    vr = torch.randn((S, H, W, D), generator=gen, device=dv).to(bf)
    n = cfg.steps
    qs = torch.randn((n, S, H, D), generator=gen, device=dv).to(bf)
    ks = torch.randn((n, S, H, D), generator=gen, device=dv).to(bf)
    vs = torch.randn((n, S, H, D), generator=gen, device=dv).to(bf)
    pos = torch.full((S,), cfg.prior + W, dtype=torch.int64, device=dv)
    y = torch.empty((S, H, D), dtype=bf, device=dv)
    kr0, vr0, A0 = kr.clone(), vr.clone(), A.clone()
    for i in range(min(warmup, n)):
        tc.tc_decode_step(qs[i], ks[i], vs[i], kr, vr, A, pos, lam, eta, g, y=y)
    st = torch.cuda.current_stream()
    runs = []
    for _ in range(3):  # n consecutive steps from the restored start state, three times
        torch.cuda.synchronize()
        kr.copy_(kr0)
        vr.copy_(vr0)
        A.copy_(A0)
        pos.fill_(cfg.prior + W)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(n):
            tc.tc_decode_step(qs[i], ks[i], vs[i], kr, vr, A, pos, lam, eta, g, y=y)
        e1.record(st)
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / n)
    ms = sorted(runs)[1]
    by = decode_bytes(S, H, D, W)
    gbs = by / (ms * 1e-3) / 1e9
    return dict(workload="decode S=%d H=%d D=%d W=%d bf16, %d consecutive steps" % (S, H, D, W, n),
                ms_per_step=ms, ms_per_step_runs=runs, steps_per_s=1e3 / ms, tokens_per_s=S * 1e3 / ms, bytes=by,
                roofline=dict(bound="hbm", achieved=gbs, peak=PEAK_HBM, unit="GB/s", frac=gbs / PEAK_HBM,
                              traffic=measured_traffic().get("decode"),
                              kernel="one tc_decode_step call (decode_kernel + pos_advance_kernel)"))


def backward_leg(steps, warmup):
    """Training backward B=4 H=16 D=128 T=8192 W=512: tc_backward per call
    (the forward that produces y and lse runs once, outside the timing)."""
    import torch

    import eviction_fed_weight_amd as tc
    import tc_inputs

    cfg = tc_inputs.CONFIGS[5]
    d = tc_inputs.prefill_inputs(5)
    dv = torch.device("cuda")
    q, k, v, dy = (torch.from_numpy(d[x]).to(dv).to(torch.bfloat16).contiguous() for x in ("q", "k", "v", "dy"))
    lam, eta, g = (torch.from_numpy(d[x]).to(dv) for x in ("lam", "eta", "gate"))
    y, _, lse = tc.tc_forward(q, k, v, lam, eta, g, cfg.W, cfg.C)
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    shape = tc.make_shape(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, cfg.C)
    ws = torch.empty(tc.tc_backward_workspace_size(shape), dtype=torch.uint8, device=dv)

    def call():
        tc.tc_backward(q, k, v, y, dy, lse, lam, eta, g, cfg.W, cfg.C, dq=dq, dk=dk, dv=dvv, ws=ws)

    ms = time_calls(call, steps, warmup)
    fl = bwd_flops(cfg.B, cfg.H, cfg.T, cfg.D, cfg.W, min(cfg.C, 64))
    tflops = fl / (ms * 1e-3) / 1e12
    return dict(workload="backward B=%d H=%d D=%d T=%d W=%d C=%d bf16" % (cfg.B, cfg.H, cfg.D, cfg.T, cfg.W, cfg.C),
                ms_per_call=ms, tokens_per_s=cfg.B * cfg.T / (ms * 1e-3), flops=fl,
                roofline=dict(bound="mfma", achieved=tflops, peak=PEAK_BF16, unit="TFLOP/s", frac=tflops / PEAK_BF16,
                              traffic=measured_traffic().get("backward"),
                              kernel="one tc_backward call (segment passes + dq_kernel + dkdv_kernel + reduce)"))


def calib_leg(steps, warmup, mib=256):
    """A plain device copy of known size (read mib MiB, write mib MiB), for
    scaling the HBM byte counters of a profiler run to bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def call():
        dst.copy_(src)

    ms = time_calls(call, steps, warmup)
    return dict(workload="device copy %d MiB -> %d MiB" % (mib, mib), bytes_read=n * 4, bytes_written=n * 4,
                ms_per_call=ms, gbs=2 * n * 4 / (ms * 1e-3) / 1e9)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _timed(fn, n=1):
    """Median wall time of n runs of fn."""
    import numpy as np

    ts = []
    for _ in range(n):
        t = time.time()
        fn()
        ts.append(time.time() - t)
    return float(np.median(ts))


def cpu_baseline():
    """The oracle (unmodified: the float64 per-token recurrence, OpenMP over
    independent (b,h) or (stream, head) pairs) timed on the host cores on
    bounded samples of the workloads, about 30 s in all; each rate is scaled
    from its sample to the whole workload (the pairs are independent and
    equal in work).  The headline entry is the long-context prefill."""
    import numpy as np

    import oracle
    import tc_inputs

    cores = oracle.num_threads()
    out = {}
    # long-context prefill: all 12 heads on all cores; one head on one thread
    c3 = tc_inputs.CONFIGS[3]
    d = tc_inputs.prefill_inputs(3)
    sec = _timed(lambda: oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], c3.W))
    oracle.set_num_threads(1)
    sec1 = _timed(lambda: oracle.forward(d["q"][:, :1], d["k"][:, :1], d["v"][:, :1], d["lam"][:1], d["eta"][:1],
                                         d["gate"][:1], c3.W)) * c3.B * c3.H
    oracle.set_num_threads(cores)
    out["long_prefill"] = dict(value=c3.B * c3.T / sec, unit="tokens/s", seconds=sec,
                               sample="the whole workload (B=1 H=12 T=32768 W=1024 D=64), one run",
                               single_thread=dict(value=c3.B * c3.T / sec1, unit="tokens/s", seconds=sec1,
                                                  sample="one head on one thread, x12"))
    del d
    # training-shape prefill: the whole batch, median of runs within 3 s; one (b,h) on one thread
    c2 = tc_inputs.CONFIGS[2]
    d = tc_inputs.prefill_inputs(2)
    f2 = lambda: oracle.forward(d["q"], d["k"], d["v"], d["lam"], d["eta"], d["gate"], c2.W)  # noqa: E731
    n2 = max(3, min(50, int(3.0 / max(_timed(f2), 1e-3))))
    sec = _timed(f2, n2)
    oracle.set_num_threads(1)
    sec1 = _timed(lambda: oracle.forward(d["q"][:1, :1], d["k"][:1, :1], d["v"][:1, :1], d["lam"][:1], d["eta"][:1],
                                         d["gate"][:1], c2.W), 3) * c2.B * c2.H
    oracle.set_num_threads(cores)
    out["prefill"] = dict(value=c2.B * c2.T / sec, unit="tokens/s", seconds=sec,
                          sample="the whole batch (B=8 H=8 T=1024 W=256 D=64), median of %d runs" % n2,
                          single_thread=dict(value=c2.B * c2.T / sec1, unit="tokens/s", seconds=sec1,
                                             sample="one (b,h) sequence on one thread, median of 3, x64"))
    # serving decode: 4 of the 64 streams (all 32 heads) for 256 consecutive steps on all cores;
    # one stream for 8 steps on one thread
    c4 = tc_inputs.CONFIGS[4]
    lam, eta, g = tc_inputs.decode_params(4, c4.H)
    ns, nsteps = 4, 256
    ins = [tc_inputs.decode_stream_inputs(4, s, c4.H, c4.D, c4.W, 16, nsteps) for s in range(ns)]
    kr = np.stack([x["ring_k"] for x in ins]).astype(np.float64)
    vr = np.stack([x["ring_v"] for x in ins]).astype(np.float64)
    A = np.zeros((ns, c4.H, c4.D, c4.D))
    pos = np.full(ns, c4.prior + c4.W, np.int64)
    qs, ks, vs = (np.stack([x[n] for x in ins], axis=1) for n in ("q", "k", "v"))

    def dec(nst, ns_):
        for t in range(nst):
            oracle.decode_step(qs[t, :ns_], ks[t, :ns_], vs[t, :ns_], kr[:ns_], vr[:ns_], A[:ns_], pos[:ns_], lam, eta, g)

    sec = _timed(lambda: dec(nsteps, ns)) / nsteps * (c4.S / ns)
    oracle.set_num_threads(1)
    sec1 = _timed(lambda: dec(8, 1)) / 8 * c4.S
    oracle.set_num_threads(cores)
    out["decode"] = dict(value=1.0 / sec, unit="steps/s", seconds_per_step=sec,
                         sample="4 of the 64 streams (all 32 heads, W=4096 D=128) for 256 consecutive steps, "
                                "scaled to 64 streams",
                         single_thread=dict(value=1.0 / sec1, unit="steps/s", seconds_per_step=sec1,
                                            sample="one stream for 8 steps on one thread, x64"))
    del ins, kr, vr, A, qs, ks, vs
    # training backward: one batch row (16 of the 64 (b,h) pairs) on all cores; one pair on one thread
    c5 = tc_inputs.CONFIGS[5]
    d = tc_inputs.prefill_inputs(5)
    sl = lambda x, n: x[:1, :n]  # noqa: E731
    sec = _timed(lambda: oracle.backward(sl(d["q"], c5.H), sl(d["k"], c5.H), sl(d["v"], c5.H), sl(d["dy"], c5.H),
                                         d["lam"], d["eta"], d["gate"], c5.W)) * c5.B
    oracle.set_num_threads(1)
    sec1 = _timed(lambda: oracle.backward(sl(d["q"], 1), sl(d["k"], 1), sl(d["v"], 1), sl(d["dy"], 1), d["lam"][:1],
                                          d["eta"][:1], d["gate"][:1], c5.W)) * c5.B * c5.H
    oracle.set_num_threads(cores)
    out["backward"] = dict(value=c5.B * c5.T / sec, unit="tokens/s", seconds=sec,
                           sample="batch row 0 (16 of the 64 (b,h) pairs, T=8192 W=512 D=128) on all cores, x4",
                           single_thread=dict(value=c5.B * c5.T / sec1, unit="tokens/s", seconds=sec1,
                                              sample="one (b,h) pair on one thread, x64"))
    head = out.pop("long_prefill")
    return dict(value=head["value"], unit=head["unit"], cores=cores, kind="oracle", sample=head["sample"],
                seconds=head["seconds"], single_thread=head["single_thread"], cpu_model=cpu_model(), legs=out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--legs", default="prefill,decode,backward,train_forward,continue,chunk_mean,delta,capacity")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the TC hot path here runs on a single GPU, with no "
              "multi-GPU mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    legs = args.legs.split(",")
    log("long prefill leg (headline) ...")
    lp = prefill_leg(3, args.steps, args.warmup)
    log("  long", json.dumps(lp))
    c3 = {"workload": lp["workload"], "B": 1, "H": 12, "D": 64, "T": 32768, "W": 1024, "C": 128}
    out = {
        "metric": "TC-layer prefill tokens/s (long-context prefill, tc_forward)",
        "value": lp["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": lp["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": c3,
        "roofline": lp["roofline"],
        "cold": lp["cold"],
    }
    if "prefill" in legs:
        log("training-shape prefill leg ...")
        pre = prefill_leg(2, args.steps, args.warmup)
        log("  prefill", json.dumps(pre))
        out["prefill"] = pre
    if "decode" in legs:
        log("decode leg ...")
        dec = decode_leg(args.steps, args.warmup)
        log("  decode", json.dumps(dec))
        out["decode"] = dec
    if "backward" in legs:
        log("backward leg ...")
        bw = backward_leg(max(3, args.steps // 5), 2)
        log("  backward", json.dumps(bw))
        out["backward"] = bw
    if "continue" in legs:
        log("chunked prefill (continuation) leg ...")
        cl = continue_leg(max(3, args.steps // 5), 2)
        log("  continue", json.dumps(cl))
        out["chunked_prefill"] = cl
    if "chunk_mean" in legs:
        log("chunk-mean shortcut leg ...")
        cm = chunk_mean_leg(args.steps, args.warmup, lp["ms_per_call"])
        log("  chunk_mean", json.dumps(cm))
        out["chunk_mean_shortcut"] = cm
    if "delta" in legs:
        log("delta-rule write leg ...")
        dl = delta_leg(args.steps, args.warmup, {3: lp["ms_per_call"], 2: out["prefill"]["ms_per_call"]}
                       if "prefill" in out else {3: lp["ms_per_call"]})
        log("  delta", json.dumps(dl))
        out["delta_rule"] = dl
    if "capacity" in legs:
        log("capacity diagnostic leg ...")
        cp = capacity_leg()
        log("  capacity", json.dumps(cp))
        out["capacity"] = cp
    if "train_forward" in legs:
        log("training-shape forward leg ...")
        tf = prefill_leg(5, max(3, args.steps // 5), 2)
        log("  train_forward", json.dumps(tf))
        out["train_forward"] = tf
    out["csrc_sha256"] = csrc_digest()
    if "calib" in legs:
        log("copy calibration leg ...")
        cb = calib_leg(args.steps, args.warmup)
        log("  calib", json.dumps(cb))
        out["calib_copy"] = cb
    if not args.no_cpu:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
