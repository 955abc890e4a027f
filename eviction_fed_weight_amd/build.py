"""Build libtc.so (the TC C-ABI library) for gfx950 with hipcc, in-tree.

    python -m eviction_fed_weight_amd.build

Each HIP source is compiled to an object in parallel, then linked into
``eviction_fed_weight_amd/libtc.so``.  All device code is compiled with
packed float32 instructions disabled and with -fno-honor-nans (the kernels
never see NaN operands; this drops the canonicalising moves around fmaxf).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtc.so")
# (source, object name, extra flags)
UNITS = [
    ("tc_api.hip", "tc_api", []),
    ("tc_forward.hip", "tc_forward_bf16", ["-DTC_FWD_F32=0"]),
    # float32 forward: matrix-core results kept in VGPRs (no AGPR accumulators)
    ("tc_forward.hip", "tc_forward_f32", ["-DTC_FWD_F32=1", "-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("tc_fwd_rows.hip", "tc_fwd_rows", []),
    ("tc_decode.hip", "tc_decode", []),
    ("tc_continue.hip", "tc_continue", []),
    # delta-rule memory path (float32 matrix-core products): results kept in VGPRs
    ("tc_delta.hip", "tc_delta", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    # bf16 backward: matrix-core results kept in VGPRs (fewer scratch spills)
    ("tc_backward.hip", "tc_backward_bf16", ["-DTC_BWD_BF16=1", "-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("tc_backward.hip", "tc_backward_f32", ["-DTC_BWD_BF16=0"]),
]
SOURCES = sorted({u[0] for u in UNITS})
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(unit) -> str:
    src, name, extra = unit
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(UNITS))) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr[-4000:])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
