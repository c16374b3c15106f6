"""Builds libllmint8.so (HIP kernels + C ABI) and the benchmark's probe library for gfx950 with
hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libllmint8.so")

SOURCES = ["prep.hip", "gemm.hip", "gemv.hip", "bwd.hip", "blockwise.hip", "fourbit.hip", "noalloc.hip",
           "api.cpp"]
# the benchmark's matrix-core rate probe: a library of its own, not part of libllmint8
PROBE_SRC = os.path.join(HERE, "bench_probe", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libllmint8_probe.so")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # quantization decisions must be the plain IEEE operations written in the source
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed to build {what}")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel), link libllmint8.so and the benchmark's
    probe library. Always recompiles."""
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="llmint8_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj], verbose, src)
            return obj

        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        _run([cc, *FLAGS, "-shared", *objs, "-o", tmp_lib], verbose, "libllmint8.so")
        os.replace(tmp_lib, LIB)
    tmp_probe = PROBE_LIB + ".tmp"
    _run([cc, *FLAGS, "-shared", PROBE_SRC, "-o", tmp_probe], verbose, "libllmint8_probe.so")
    os.replace(tmp_probe, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
