"""Helpers for the GPU parity tests (device transfer, error metric, tolerances)."""
import numpy as np
import torch

# Parity bars: relative L2 error against the float64 oracle run on the same
# (bf16-rounded) inputs, over the whole tensor ...
TOL = {"f32": 1e-5, "bf16": 5e-3}
# ... and, for every tensor of per-token rows, the worst single row: max over
# rows of ||row - ref row|| / max(||ref row||, median row norm).  Rows at
# least as large as the median are measured against their own norm; smaller
# rows (a gradient row is small by cancellation, the first rows of dq are 0
# exactly) against the median norm, because their rounding errors scale with
# the size of their terms, not of their sum.  A correct bf16 row carries the
# bf16 rounding of its output (about 1.1e-3 relative rms, the largest of
# thousands of 64-element rows about 2.5e-3) and of the probabilities; a row
# off by 2 % of its size (or of the median size) is a fault that the
# whole-tensor norm hides at 10^5-10^6 rows (one wholly wrong row in 524,288
# moves it by 1.4e-3).
ROWTOL = {"f32": 1e-4, "bf16": 2e-2}


def bar(key: str, dtype: str) -> float:
    """The bar of an error entry: keys ending in "_row" are worst-row errors."""
    return ROWTOL[dtype] if key.endswith("_row") else TOL[dtype]


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype="f32"):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdtype(dtype)).contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def rowrel(a, b, per_element=False) -> float:
    """Worst relative L2 error of one row (the last axis), or of one element
    (per_element: for per-token scalars such as lse).  A reference row of
    norm below the median row norm is measured against the median instead
    of its own norm: a row that is small by cancellation (a gradient row,
    say) carries rounding errors of the size of its terms, not of its sum,
    and an all-zero row cannot divide by zero.  A wholly wrong row of
    typical size still scores about 1."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if per_element or a.ndim == 1:
        a = a.reshape(-1, 1)
        b = b.reshape(-1, 1)
    else:
        a = a.reshape(-1, a.shape[-1])
        b = b.reshape(-1, b.shape[-1])
    nb = np.linalg.norm(b, axis=1)
    floor = max(float(np.median(nb)), 1e-30)
    return float(np.max(np.linalg.norm(a - b, axis=1) / np.maximum(nb, floor)))


def errors(**pairs) -> dict:
    """Whole-tensor and worst-row errors of (gpu, reference) pairs: name ->
    rel, name_row -> rowrel ("lse" per element)."""
    out = {}
    for name, (a, b) in pairs.items():
        out[name] = rel(a, b)
        out[name + "_row"] = rowrel(a, b, per_element=(name == "lse"))
    return out


def say(*a):
    print(*a, flush=True)
