"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code,
run on the CPU: the CPU oracle (oracle/tc_oracle.c, every entry point on
small edge-case inputs) and the library's host-side validation and
workspace planning (eviction_fed_weight_amd/csrc/tc_api.hip, with the kernel
launchers replaced by stubs that abort).  The sanitizers are applied to host
code only: each -fsanitize option on a hipcc line is preceded by -Xarch_host,
so no device code is built with them."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-g", "-O1", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "tc_oracle.c"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", exe, "-lm"])
    r = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert r.stdout.strip().endswith("ok")


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not available")
    api = str(tmp_path / "api_san.o")
    drv = str(tmp_path / "abi_check.o")
    exe = str(tmp_path / "abi_san")
    base = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include")]
    run(base + HOST_SAN + ["-c", os.path.join(ROOT, "eviction_fed_weight_amd", "csrc", "tc_api.hip"), "-o", api])
    run(base + HOST_SAN + ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_check.cpp"), "-o", drv])
    run([CLANGXX, "-fsanitize=address,undefined", drv, api, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = run([exe], env=ENV)
    assert r.stdout.strip().endswith("ok")
