"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: outlier set, int8 codes, row/column statistics and int32 accumulators
bit-exact; Y within max-abs-relative 1e-3 (``oracle.parity_error``) and finite.
Small cases compare every element; the full-size workloads compare all of the
quantization stages and the C/Y rows of a seeded sample of rows.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu

Y_TOL = 1e-3
GEMM, GEMV, AUTO = m8.LLMINT8_PATH_GEMM, m8.LLMINT8_PATH_GEMV, m8.LLMINT8_PATH_AUTO


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m8.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize_weight_checked(W):
    """GPU weight quantization, checked bit-exact against the oracle."""
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    Wd = _dev(W)
    Wq, sW = m8.llmint8_quantize_weight(Wd)
    assert np.array_equal(_host(Wq), Wq_ref), "Wq differs"
    assert np.array_equal(_host(sW).view(np.uint32), sW_ref.view(np.uint32)), "sW differs"
    del Wd
    return Wq, sW, Wq_ref, sW_ref


def run_case(name, W, X, thr, path, rows=None, check_auto=False):
    """Run one forward on the GPU and compare every stage with the oracle."""
    T, K = X.shape
    N = W.shape[0]
    _say(f"{name}: T={T} K={K} N={N} thr={thr} path={path}")
    Wq, sW, Wq_ref, sW_ref = quantize_weight_checked(W)
    Xd = _dev(X)
    full = rows is None
    out = m8.llmint8_linear_debug(Xd, Wq, sW, thr, path=path, want_C=True)
    st = oracle.linear(X, Wq_ref, sW_ref, thr, rows=None if full else rows)
    count = int(_host(out["count"])[0])
    assert count == st.count, (count, st.count)
    assert np.array_equal(_host(out["bitmap"]).view(np.uint32), st.bitmap)
    assert np.array_equal(_host(out["idx"])[:count], st.idx)
    assert np.array_equal(_host(out["Xq"]), st.Xq), "Xq differs"
    assert np.array_equal(_host(out["aX"]).view(np.uint32), st.aX.view(np.uint32)), "aX differs"
    C = _host(out["C"])
    Y = _host(out["Y"])
    sel = slice(None) if full else rows
    assert np.array_equal(C[sel], st.C), "C differs"
    err = oracle.parity_error(Y[sel], st.Y)
    assert err <= Y_TOL, f"Y parity error {err}"     # also: non-finite only where the oracle is
    if check_auto:
        Y2 = m8.llmint8_linear(Xd, Wq, sW, thr)
        assert np.array_equal(_host(Y2).view(np.uint16), Y.view(np.uint16)), "plain call differs"
    return err, count


def _rng(seed):
    return np.random.default_rng(seed)


def _small(T, K, N, seed, n_out=3, lo=20.0, hi=60.0, sigma=0.05):
    w = workloads.Workload("edge", T=T, K=K, N=N, sigma=sigma, n_out=min(n_out, K), lo=lo, hi=hi,
                           threshold=6.0, seed=seed)
    W, X, _, _ = workloads.make(w)
    return W, X


# --------------------------------------------------------------------------- small, full compare

@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_tiny_workload(path):
    w = workloads.CONFIGS["tiny"]
    W, X, _, _ = workloads.make(w)
    run_case("tiny", W, X, w.threshold, path, check_auto=True)


@pytest.mark.parametrize("T", [1, 2, 3, 7, 9, 16, 17, 33, 130, 300])
def test_ragged_rows(T):
    W, X = _small(T, 256, 200, seed=100 + T)
    for path in ([GEMM, GEMV] if T <= 16 else [GEMM]):
        run_case(f"ragged T={T}", W, X, 6.0, path, check_auto=True)


@pytest.mark.parametrize("K,N", [(16, 1), (48, 3), (1040, 17), (4112, 250), (272, 1000), (8192, 64)])
def test_ragged_k_and_n(K, N):
    W, X = _small(37, K, N, seed=K + N)
    run_case(f"ragged K={K} N={N}", W, X, 6.0, GEMM)
    run_case(f"ragged K={K} N={N} gemv", W, X[:5], 6.0, GEMV)


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_no_outliers_and_infinite_threshold(path):
    W, X = _small(12, 512, 96, seed=7)
    run_case("thr=inf", W, X, math.inf, path)
    X2 = np.clip(X.astype(np.float32), -5, 5).astype(np.float16)
    _, c = run_case("no outlier", W, X2, 6.0, path)
    assert c == 0


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_every_column_outlier(path):
    rng = _rng(3)
    X = workloads.random_fp16(rng, (9, 96), 2.0)
    X[X == 0] = np.float16(0.5)
    W = workloads.random_fp16(rng, (40, 96), 0.05)
    _, c = run_case("all columns", W, X, 1e-3, path)
    assert c == 96


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_threshold_ties_and_zero_rows(path):
    rng = _rng(5)
    X = workloads.random_fp16(rng, (11, 160), 1.0)
    X = np.clip(X.astype(np.float32), -5.5, 5.5).astype(np.float16)
    X[2, 17] = np.float16(6.0)            # exactly the threshold: an outlier
    X[4, 33] = np.float16(-6.0)
    X[5, 70] = np.float16(5.99609375)     # just below: not an outlier
    X[7] = 0                              # an all-zero row
    X[8, :] = np.float16(2.5)             # equal values: rounding ties after scaling
    W = workloads.random_fp16(rng, (72, 160), 0.05)
    W[3] = 0                              # an all-zero weight row
    _, c = run_case("ties", W, X, 6.0, path)
    assert c == 2


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_single_outlier_column(path):
    rng = _rng(6)
    X = np.clip(workloads.random_fp16(rng, (13, 384), 1.0).astype(np.float32), -5, 5).astype(np.float16)
    X[6, 201] = np.float16(-37.5)                 # |O| = 1, in one row only
    W = workloads.random_fp16(rng, (88, 384), 0.05)
    _, c = run_case("|O|=1", W, X, 6.0, path)
    assert c == 1


@pytest.mark.parametrize("tile", sorted(m8.LLMINT8_PATH_GEMM_TILES))
def test_every_gemm_tile_ragged(tile):
    """Each GEMM tile, forced, on ragged T, K and N: partial tiles along both
    output axes, a K tail, no outliers, one chunk and several chunks."""
    path = m8.LLMINT8_PATH_GEMM_TILES[tile]
    for (T, K, N, n_out, seed) in ((300, 1040, 1000, 3, 1), (257, 4096, 705, 0, 2),
                                   (64, 272, 360, 40, 3), (513, 640, 2100, 100, 4),
                                   (1, 16, 3, 1, 5), (33, 48, 353, 2, 6), (5, 65536, 40, 20, 7)):
        W, X = _small(T, K, N, seed=seed, n_out=n_out)
        # every tile computes each output element with the same operations:
        # where the plain call also takes the GEMM (tile by cost), it must give the same bits
        _, c = run_case(f"tile {tile}", W, X, 6.0 if n_out else math.inf, path,
                        check_auto=T > m8.llmint8_gemv_max_rows(K))
        assert (c > 0) == (n_out > 0)


def test_integer_inputs_quantize_exactly():
    rng = _rng(9)
    X = rng.integers(-127, 128, size=(20, 128)).astype(np.float16)
    W = rng.integers(-127, 128, size=(48, 128)).astype(np.float16)
    X[:, 0] = 127
    W[:, 0] = -127
    for path in (GEMM,):
        run_case("integer", W, X, math.inf, path)


def test_many_outlier_chunks():
    W, X = _small(70, 1024, 300, seed=21, n_out=100)
    _, c = run_case("100 outliers", W, X, 6.0, GEMM)
    assert c >= 100
    run_case("100 outliers gemv", W, X[:9], 6.0, GEMV)


def test_repeat_calls_bit_identical():
    W, X = _small(300, 1024, 520, seed=31, n_out=9)
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Xd = _dev(X)
    ws = torch.empty((m8.llmint8_workspace_bytes(300, 1024, 520),), dtype=torch.uint8, device="cuda")
    ys = [_host(m8.llmint8_linear(Xd, Wq, sW, 6.0, workspace=ws)).view(np.uint16) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_int8linear_module_and_memory():
    W, X = _small(24, 512, 128, seed=41)
    layer = m8.Int8Linear(_dev(W), threshold=6.0)
    Y = _host(layer(_dev(X).reshape(2, 12, 512)))
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq_ref, sW_ref, 6.0)
    assert oracle.parity_error(Y.reshape(24, 128), st.Y) <= Y_TOL
    assert layer.memory_bytes() == 128 * 512 + 4 * 128


def test_timed_entry_records_kernel_events():
    W, X = _small(256, 1024, 512, seed=51)
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Xd = _dev(X)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    ws = torch.empty((m8.llmint8_workspace_bytes(256, 1024, 512),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((256, 512), dtype=torch.float16, device="cuda")
    nk = m8.llmint8_linear_timed(Xd, Wq, sW, 6.0, Y, ws, ev, path=GEMM)
    torch.cuda.synchronize()
    assert nk == 3
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(3))
    Y2 = m8.llmint8_linear(Xd, Wq, sW, 6.0, workspace=ws)
    assert np.array_equal(_host(Y).view(np.uint16), _host(Y2).view(np.uint16))


# --------------------------------------------------------------------------- full-size workloads

def _sample_rows(T, n, seed):
    r = _rng(seed)
    rows = np.sort(r.choice(T, size=min(n, T), replace=False))
    return np.unique(np.concatenate([rows, [0, T - 1]]))


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_workload(T):
    w = workloads.CONFIGS["decode"]
    W, X, _, _ = workloads.make(w, T=T)
    run_case(f"decode T={T}", W, X, w.threshold, GEMV, check_auto=True)
    run_case(f"decode T={T} gemm", W, X, w.threshold, GEMM)


def test_prefill_workload():
    w = workloads.CONFIGS["prefill"]
    W, X, _, _ = workloads.make(w)
    err, c = run_case("prefill", W, X, w.threshold, AUTO, rows=_sample_rows(w.T, 48, 1))
    assert c >= w.n_out


def test_large_workload():
    w = workloads.CONFIGS["large"]
    W, X, cols, zrows = workloads.make(w)
    rows = np.unique(np.concatenate([_sample_rows(w.T, 24, 2), zrows[:4]]))
    err, c = run_case("large", W, X, w.threshold, AUTO, rows=rows)
    assert c >= w.n_out


@pytest.mark.parametrize("n_out", workloads.SWEEP_N_OUT)
def test_sweep_workload(n_out):
    w = workloads.CONFIGS["sweep"].with_(n_out=n_out)
    W, X, _, _ = workloads.make(w)
    for thr in workloads.SWEEP_THRESHOLDS:
        run_case(f"sweep n_out={n_out}", W, X, thr, AUTO, rows=_sample_rows(w.T, 16, 3 + n_out))


# --------------------------------------------------------------------------- limits

def test_maximum_k():
    """K = 65536, the largest K the library takes: the bitmap prefix tables fill
    LDS and no rows fit the fused decode kernel, so every T goes to the GEMM."""
    assert m8.llmint8_gemv_max_rows(65536) == 0
    W, X = _small(5, 65536, 72, seed=65, n_out=20)
    _, c = run_case("K=65536", W, X, 6.0, AUTO, check_auto=True)
    assert c >= 20


def test_many_outliers_at_large_k():
    """|O| in the thousands: the gather beyond the LDS index table (binary search
    over the bitmap prefix) and 32-column chunks far apart."""
    rng = _rng(66)
    X = workloads.random_fp16(rng, (9, 16384), 1.0)
    X[3, ::3] = np.float16(9.0)                     # 5462 outlier columns
    W = workloads.random_fp16(rng, (40, 16384), 0.02)
    _, c = run_case("|O|=5462", W, X, 6.0, GEMM)
    assert c >= 5461
