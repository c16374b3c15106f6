"""Seeded random sweep of the forward on the GPU against the oracle: shapes,
outlier counts, thresholds, both 16-bit types, with and without bias, and every
route (the cost model's choice, the fused decode kernel, the GEMM with its own
tile or a forced one). Every case compares every stage as the other parity
tests do (outlier set, codes, statistics and C bit-exact; Y within the bar of
its type)."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402
from test_gpu_bf16 import GEMM, GEMV, AUTO, _as, _bias, _small, run_case  # noqa: E402

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("LLMINT8_SWEEP_CASES", "160"))  # more for a longer soak
TILES = sorted(m8.LLMINT8_PATH_GEMM_TILES.values())


def _case(i):
    rng = np.random.default_rng(7000 + i)
    small_t = rng.random() < 0.35
    T = int(rng.integers(1, 17)) if small_t else int(rng.integers(17, 700))
    K = 16 * int(rng.integers(1, 401))
    N = int(rng.integers(1, 1500))
    N = max(1, min(N, int(1.5e9 // (T * K))))
    n_out = int(rng.choice([0, 1, 3, 17, 40, 100]))
    thr = math.inf if rng.random() < 0.1 else 6.0
    dtype = "bf16" if rng.random() < 0.5 else "f16"
    bias = rng.random() < 0.5
    path = int(rng.choice([AUTO, GEMM] + TILES))
    if T <= m8.llmint8_gemv_max_rows(K) and rng.random() < 0.5:
        path = GEMV
    return T, K, N, n_out, thr, dtype, bias, path


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m8.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    T, K, N, n_out, thr, dtype, bias, path = _case(i)
    W, X = _as(dtype, *_small(T, K, N, seed=9000 + i, n_out=n_out))
    b = _bias(9000 + i, N, dtype, on=bias)
    _, c = run_case(f"sweep {i}", W, X, thr, path, dtype, bias=b, check_plain=path == AUTO)
    if thr == math.inf:
        assert c == 0
