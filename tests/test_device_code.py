"""The gfx950 code of every kernel source, compiled as the build compiles it,
holds no packed fp32 arithmetic (the build turns the compiler's use of it off)
and no store, atomic or write-back through the scalar data cache (every kernel
writes through vector memory instructions). Checked on the assembly, on the CPU.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixed_precision_int8_amd")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("prep.hip", "gemm.hip", "gemv.hip", "bwd.hip",
                                                  "blockwise.hip", "fourbit.hip", "noalloc.hip")]
SOURCES.append(os.path.join(PKG, "bench_probe", "probe.hip"))

PACKED_FP32 = re.compile(r"^\s*v_pk_(add|mul|fma|mov)_(f32|b32)\b", re.M)
SCALAR_WRITE = re.compile(r"^\s*s_(store|buffer_store|atomic|buffer_atomic|scratch_store|dcache_wb|dcache_discard)", re.M)


def test_no_packed_fp32_or_scalar_writes_in_device_code():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    from mixed_precision_int8_amd import build
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    with tempfile.TemporaryDirectory() as tmp:
        def asm(src):
            out = os.path.join(tmp, os.path.basename(src) + ".s")
            r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                                "-I", os.path.join(PKG, "csrc"), src, "-o", out], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return src, open(out).read()
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(asm, SOURCES))
    for src, text in results:
        if not src.endswith("noalloc.hip"):  # that file holds the static scratch only
            assert "s_endpgm" in text, f"{os.path.basename(src)}: no kernel code"
        m = PACKED_FP32.search(text)
        assert m is None, f"{os.path.basename(src)}: {m.group(0).strip()}"
        m = SCALAR_WRITE.search(text)
        assert m is None, f"{os.path.basename(src)}: {m.group(0).strip()}"
