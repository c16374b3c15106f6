"""The host code of the C ABI (argument validation, workspace sizing, tile and
row queries, code books) under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled as for the product (gfx950 device code
included, though nothing here launches) with the sanitizers on the host pass
only, linked with the C driver tests/host_check.c and run on the CPU. Any
sanitizer report aborts the C driver.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_int8_amd", "csrc")
SOURCES = ["prep.hip", "gemm.hip", "gemv.hip", "bwd.hip", "blockwise.hip", "fourbit.hip", "noalloc.hip",
           "api.cpp"]
# each sanitizer flag goes to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name):
    for c in (os.path.join("/opt/rocm/bin", name), os.path.join("/opt/rocm/llvm/bin", name),
              shutil.which(name)):
        if c and os.path.exists(c):
            return c
    return None


def test_host_paths_under_sanitizers():
    hipcc, clang = _tool("hipcc"), _tool("clang")
    if not hipcc or not clang:
        pytest.skip("ROCm compilers not found")
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            out = os.path.join(tmp, os.path.basename(src) + ".o")
            r = subprocess.run([hipcc, "--offload-arch=gfx950", "-c", "-O1", "-g", "-std=c++17",
                                "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                                "-packed-fp32-ops", *SAN, "-I", os.path.join(ROOT, "include"),
                                "-I", CSRC, os.path.join(CSRC, src), "-o", out],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return out
        with ThreadPoolExecutor(max_workers=4) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        drv = os.path.join(tmp, "host_check.o")
        r = subprocess.run([clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                            "-I", os.path.join(ROOT, "include"),
                            "-c", os.path.join(ROOT, "tests", "host_check.c"), "-o", drv],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(tmp, "host_check")
        r = subprocess.run([hipcc, *SAN, *objs, drv, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0 and "host check ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
