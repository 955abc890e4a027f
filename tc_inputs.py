"""Seeded synthetic inputs for the TC layer (shared by tests, bench and smoke).

This module only draws random numbers and rounds them to the storage dtype;
it contains none of the layer's arithmetic.  Both the GPU library and the CPU
oracle read the exact bytes produced here.

Workloads (the pages give no shapes; these stand in for the settings the
pages describe -- training context 1,024, evaluation at 32x that context,
batched serving decode, training backward):

  1  tiny fp32:   B=1  H=1  D=16  T=64     W=8     C=8    lam=.9 eta=.5 g=0
  2  prefill:     B=8  H=8  D=64  T=1024   W=256   C=64   bf16
  3  long:        B=1  H=12 D=64  T=32768  W=1024  C=128  bf16, 5% planted
                  key repeats more than W apart (associative-recall pairs)
  4  decode:      S=64 streams, H=32, D=128, W=4096, bf16 ring, 1024 steps
  5  backward:    B=4  H=16 D=128 T=8192   W=512   C=64   bf16, dy ~ N(0,1)

Per-head parameters (2-5): lam = sigmoid(U(2,5)), eta = sigmoid(U(-3,0)),
g ~ N(0,1), kept as float32 values.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    D: int
    T: int
    W: int
    C: int
    dtype: str  # "f32" or "bf16"
    qkv_std: float
    S: int = 0  # decode streams (config 4)
    steps: int = 0  # decode steps (config 4)
    prior: int = 0  # prior evictions in the decode start state (config 4)


CONFIGS = {
    1: Config("tiny_fp32", 1, 1, 16, 64, 8, 8, "f32", 1.0),
    2: Config("prefill_b8h8_t1k", 8, 8, 64, 1024, 256, 64, "bf16", 1.0 / 8.0),
    3: Config("long_prefill_h12_t32k", 1, 12, 64, 32768, 1024, 128, "bf16", 1.0 / 8.0),
    4: Config("decode_s64h32_w4k", 64, 32, 128, 0, 4096, 0, "bf16", 1.0, S=64, steps=1024, prior=8192),
    5: Config("backward_b4h16_t8k", 4, 16, 128, 8192, 512, 64, "bf16", 1.0 / np.sqrt(128.0)),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 arrays holding exactly representable bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def head_params(rng_l, rng_e, rng_g, H: int):
    lam = (1.0 / (1.0 + np.exp(-rng_l.uniform(2.0, 5.0, H)))).astype(np.float32)
    eta = (1.0 / (1.0 + np.exp(-rng_e.uniform(-3.0, 0.0, H)))).astype(np.float32)
    gate = rng_g.standard_normal(H).astype(np.float32)
    return lam, eta, gate


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.asarray(x, np.float32)


def plant_pairs(k: np.ndarray, W: int, frac: float, rng) -> np.ndarray:
    """Associative-recall plants (in place on k [B,H,T,D]): per head, round(frac*T)
    sources i (without replacement) in [0, T-W-2], each copied to a
    destination j uniform in [i+W+1, T-1] (redrawn on collision).
    Returns the (b, h, i, j) list."""
    B, H, T, _ = k.shape
    n = int(round(frac * T))
    out = []
    for b in range(B):
        for h in range(H):
            src = rng.choice(T - W - 1, size=n, replace=False)
            used = set(int(s) for s in src)
            for i in src:
                i = int(i)
                while True:
                    j = int(rng.integers(i + W + 1, T))
                    if j not in used:
                        break
                used.add(j)
                k[b, h, j] = k[b, h, i]
                out.append((b, h, i, j))
    return np.asarray(out, dtype=np.int64)


def prefill_inputs(cfg_id: int, seed: int | None = None, *, B=None, H=None, T=None, D=None,
                   W=None, dtype=None, with_dy=None, plants=None):
    """Inputs of a prefill/backward workload as float32 numpy arrays holding
    the exact stored values.  Shape overrides give smaller cases drawn the
    same way.  Returns a dict with q, k, v, lam, eta, gate (and dy)."""
    cfg = CONFIGS[cfg_id]
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    T = cfg.T if T is None else T
    D = cfg.D if D is None else D
    W = cfg.W if W is None else W
    dtype = cfg.dtype if dtype is None else dtype
    with_dy = (cfg_id == 5) if with_dy is None else with_dy
    plants = (cfg_id == 3) if plants is None else plants
    seed = cfg_id if seed is None else seed
    r = _streams(seed, 8)
    shape = (B, H, T, D)
    std = cfg.qkv_std if cfg_id != 1 else 1.0
    q = _store(r[0].standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)
    k = _store(r[1].standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)
    v = _store(r[2].standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)
    if cfg_id == 1:
        lam = np.full(H, 0.9, np.float32)
        eta = np.full(H, 0.5, np.float32)
        gate = np.zeros(H, np.float32)
    else:
        lam, eta, gate = head_params(r[3], r[4], r[5], H)
    out = dict(q=q, k=k, v=v, lam=lam, eta=eta, gate=gate, W=W, dtype=dtype)
    if with_dy:
        out["dy"] = _store(r[6].standard_normal(shape, dtype=np.float32), dtype)
    if plants and T > W + 2:
        out["plants"] = plant_pairs(out["k"], W, 0.05, r[7])
    return out


def decode_params(seed: int = 4, H: int = 32):
    r = _streams(seed, 8)
    return head_params(r[3], r[4], r[5], H)


def decode_stream_inputs(seed: int, s: int, H: int, D: int, W: int, prior: int, steps: int,
                         dtype: str = "bf16"):
    """Per-stream draw for the decode workload (stream s independent of the
    others, so sampled streams can be regenerated alone):
      prior_k, prior_v [H, prior, D]  -- pairs evicted before the start
      ring_k, ring_v   [H, W, D]      -- the W pairs resident in the ring
      q, k, v          [steps, H, D]  -- the new tokens of each step
    Everything N(0,1), rounded to the storage dtype."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000 + s])))
    f = lambda *shape: _store(g.standard_normal(shape, dtype=np.float32), dtype)  # noqa: E731
    prior_k = f(H, prior, D)
    prior_v = f(H, prior, D)
    ring_k = f(H, W, D)
    ring_v = f(H, W, D)
    q = f(steps, H, D)
    k = f(steps, H, D)
    v = f(steps, H, D)
    return dict(prior_k=prior_k, prior_v=prior_v, ring_k=ring_k, ring_v=ring_v, q=q, k=k, v=v)


def capacity_inputs(N: int, D: int, H: int = 4, seed: int = 6, dtype: str = "bf16", orthonormal: bool = False):
    """Raw associative-memory capacity probe.  The abstract of "Tensor Cache:
    Eviction-conditioned Associative Memory for Transformers" lists
    memory-capacity diagnostics among its experiments; its technical summary
    (results) reports only that retrieval falls as more unrelated associations
    share the fixed state, with no parameters, so this probe is one reading of
    it.  One
    sequence of 2N tokens per head, for a layer with window W = 1, lambda =
    eta = 1 and a gate logit of 30 (sigmoid = 1 in float32):
      tokens 0 .. N-1    write pairs: q = 0, k = k_i (unit norm), v = v_i ~ N(0,1)
      tokens N .. 2N-1   reads:       q = k_i, k = 0, v = 0
    With W = 1 every pair leaves the window one step after it enters, so row
    N + i reads the memory of all N pairs with the key of pair i (the read
    tokens write zero outer products and their own window value is zero).
    orthonormal=True (N <= D) draws orthonormal keys.  Returns q, k, v
    [1, H, 2N, D] in the storage dtype (as float32 arrays), lam, eta, gate [H]
    and the stored values [H, N, D]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, N, D])))
    if orthonormal:
        assert N <= D
        keys = np.stack([np.linalg.qr(g.standard_normal((D, D)))[0][:, :N].T for _ in range(H)]).astype(np.float32)
    else:
        keys = g.standard_normal((H, N, D), dtype=np.float32)
        keys /= np.linalg.norm(keys, axis=-1, keepdims=True)
    keys = _store(keys, dtype)
    vals = _store(g.standard_normal((H, N, D), dtype=np.float32), dtype)
    z = np.zeros((H, N, D), np.float32)
    q = np.concatenate([z, keys], axis=1)[None]
    k = np.concatenate([keys, z], axis=1)[None]
    v = np.concatenate([vals, z], axis=1)[None]
    ones = np.ones(H, np.float32)
    return q, k, v, ones, ones.copy(), np.full(H, 30.0, np.float32), vals
