"""Helpers for the GPU parity tests (device transfer, error metric, tolerances)."""
import numpy as np
import torch

# Parity bars: relative L2 error against the float64 oracle run on the same
# (bf16-rounded) inputs.
TOL = {"f32": 1e-5, "bf16": 5e-3}


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


def say(*a):
    print(*a, flush=True)
