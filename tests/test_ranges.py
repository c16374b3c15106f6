"""Size limits of the C ABI against the buffer windows of the kernels (CPU).

The kernels read ragged edges through buffer loads whose "reads as zero"
offset is 2^31, which is only out of range while a window spans at most 2^31
bytes. ``tests/range_check.cpp`` sweeps every admission limit (and the shapes
on both sides of it) with the library's own admission and window functions
(``csrc/ranges.h``), built on the host and run without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_admitted_shapes_keep_every_window_within_2_31_bytes():
    hipcc = next((c for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")) if c and os.path.exists(c)),
                 None)
    if hipcc is None:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "range_check")
        r = subprocess.run([hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "range_check.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and "ranges ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
        print(r.stdout.strip())
