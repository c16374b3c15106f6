"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: outlier set, int8 codes, row/column statistics and int32 accumulators
bit-exact; Y within max-abs-relative 1e-3 (``oracle.parity_error``) and finite.
Every case, the full-size workloads included, compares every element of every
stage (C and Y over all rows).
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


@pytest.mark.parametrize("T,K,N", [(11, 1040, 70), (16, 2032, 33), (13, 16, 9), (15, 528, 100), (9, 2048, 48)])
def test_sixteen_row_form_ragged(T, K, N):
    """The fused kernel's 16-row form (K up to 2048) hands out one (row,
    chunk) item per thread: row counts and chunk counts that do not divide
    the 512 threads, and one row group of 16 rows."""
    W, X = _small(T, K, N, seed=7 * T + K, n_out=4)
    run_case(f"16-row form T={T} K={K} N={N}", W, X, 6.0, GEMV)


@pytest.mark.parametrize("K,N", [(16, 1), (48, 3), (1040, 17), (4112, 250), (272, 1000), (8192, 64)])
def test_ragged_k_and_n(K, N):
    W, X = _small(37, K, N, seed=K + N)
    run_case(f"ragged K={K} N={N}", W, X, 6.0, GEMM)
    run_case(f"ragged K={K} N={N} gemv", W, X[:5], 6.0, GEMV)


@pytest.mark.parametrize("T,K,N", [(37, 8208, 40), (300, 12304, 96), (33, 16384, 33), (1, 14336, 17)])
def test_long_rows_one_register_buffer(T, K, N):
    """Rows of 8193 to 16384 columns: the activation quantization holds a row in
    one register buffer of 32 chunks per lane (shorter rows take two buffers,
    longer ones two passes over memory); every stage bit-exact."""
    W, X = _small(T, K, N, seed=K + T, n_out=5)
    run_case(f"long rows K={K}", W, X, 6.0, GEMM, check_auto=T > 16)


def test_long_rows_several_per_wavefront():
    """T past 4096 with rows of 8193 to 16384 columns: on a 256-CU device each
    quantization wavefront takes two rows through its single register buffer,
    loading the second after the first is stored; every stage bit-exact."""
    W, X = _small(4500, 8320, 40, seed=4501, n_out=6)
    run_case("long rows, several per wavefront", W, X, 6.0, GEMM, check_auto=True)


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


@pytest.mark.parametrize("T,K,n_out", [(3, 8192, 45), (8, 4096, 32), (1, 14336, 33), (12, 4096, 40),
                                       (16, 2048, 20), (6, 2064, 9), (11, 3056, 14), (2, 10000, 36),
                                       (4, 10016, 7)])
def test_gemv_outlier_bytes_across_k_ranges(T, K, n_out):
    """Decode kernel: outlier columns spread over each of the four K
    quarters and every register batch (two at K = 8192, four at 14336), more
    than one 32-column chunk of them, ragged N; every form of the X work:
    X held in registers (up to 8 rows and K <= 8192, 4096 at 8 rows; 16 rows
    with K <= 2048), X copied to LDS and worked by the X wavefronts alone
    (K a multiple of 2048 past those sizes), and by all 8 wavefronts (3056,
    10000, 10016). Bit-exact stages and Y within the bar."""
    W, X = _small(T, K, 300, seed=K + n_out, n_out=n_out)
    _, c = run_case(f"gemv outliers over K ranges K={K}", W, X, 6.0, GEMV)
    assert c >= n_out


def test_repeat_calls_bit_identical():
    W, X = _small(300, 1024, 520, seed=31, n_out=9)
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Xd = _dev(X)
    ws = torch.empty((m8.llmint8_workspace_bytes(300, 1024, 520),), dtype=torch.uint8, device="cuda")
    ys = [_host(m8.llmint8_linear(Xd, Wq, sW, 6.0, workspace=ws)).view(np.uint16) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


# --------------------------------------------------------------------------- workspace reuse

def _check_stages(out, st, name):
    count = int(_host(out["count"])[0])
    assert count == st.count, (name, count, st.count)
    assert np.array_equal(_host(out["bitmap"]).view(np.uint32), st.bitmap), name
    assert np.array_equal(_host(out["idx"])[:count], st.idx), name
    assert np.array_equal(_host(out["Xq"]), st.Xq), f"{name}: Xq differs"
    assert np.array_equal(_host(out["aX"]).view(np.uint32), st.aX.view(np.uint32)), f"{name}: aX differs"
    err = oracle.parity_error(_host(out["Y"]), st.Y)
    assert err <= Y_TOL, f"{name}: Y parity error {err}"


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_forward_any_workspace_contents(fill):
    """Whatever the workspace holds on entry, the stages are the oracle's: every
    region a call reads (the scan's partial bitmaps included) is written by that
    call first."""
    T, K, N = 520, 2048, 300
    W, X = _small(T, K, N, seed=61, n_out=5)
    _say(f"workspace filled with {fill}: T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = quantize_weight_checked(W)
    st = oracle.linear(X, Wq_ref, sW_ref, 6.0)
    nb = m8.llmint8_workspace_bytes(T, K, N)
    if fill == "zeros":
        ws = torch.zeros((nb,), dtype=torch.uint8, device="cuda")
    elif fill == "ones":
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    else:
        ws = _dev(_rng(62).integers(0, 256, size=nb, dtype=np.uint8))
    for rep in range(2):
        out = m8.llmint8_linear_debug(_dev(X), Wq, sW, 6.0, path=GEMM, workspace=ws, want_C=False)
        _check_stages(out, st, f"{fill} call {rep}")


def test_forward_alternating_inputs_one_workspace():
    """Calls in order on one workspace with inputs whose outlier columns differ:
    no call takes anything (partial bitmaps, outlier operands) from an earlier one."""
    T, K, N = 700, 1024, 200
    W, X0 = _small(T, K, N, seed=71, n_out=4)
    Xs = [X0] + [_small(T, K, N, seed=sd, n_out=4)[1] for sd in (72, 73)]
    _say(f"alternating inputs: T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = quantize_weight_checked(W)
    sts = [oracle.linear(X, Wq_ref, sW_ref, 6.0) for X in Xs]
    assert len({tuple(st.idx) for st in sts}) == 3
    ws = torch.empty((m8.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        for i, (X, st) in enumerate(zip(Xs, sts)):
            out = m8.llmint8_linear_debug(_dev(X), Wq, sW, 6.0, path=GEMM, workspace=ws, want_C=False)
            _check_stages(out, st, f"input {i}, pass {rep}")


def test_forward_graph_replays_new_inputs():
    """One call captured in a HIP graph and replayed with new data in the same X
    buffer (copied in by eager work between replays): every replay decides the
    outlier set of its own X, bit-identical to an eager call."""
    T, K, N = 520, 2048, 300
    W, X0 = _small(T, K, N, seed=81, n_out=5)
    Xs = [X0] + [_small(T, K, N, seed=sd, n_out=5)[1] for sd in (82, 83)]
    _say(f"graph replays: T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = quantize_weight_checked(W)
    sts = [oracle.linear(X, Wq_ref, sW_ref, 6.0) for X in Xs]
    nb = m8.llmint8_workspace_bytes(T, K, N)
    Xd = _dev(X0)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
    ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty((nb,), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m8.llmint8_linear(Xd, Wq, sW, 6.0, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m8.llmint8_linear(Xd, Wq, sW, 6.0, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, (X, st) in enumerate(zip(Xs, sts)):
            Xd.copy_(torch.from_numpy(X))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            Yg = _host(Y).copy()
            Ye = _host(m8.llmint8_linear(Xd, Wq, sW, 6.0, workspace=ws2))
            assert np.array_equal(Yg.view(np.uint16), Ye.view(np.uint16)), f"replay {rep}/{i} differs"
            err = oracle.parity_error(Yg, st.Y)
            assert err <= Y_TOL, f"replay {rep}/{i}: Y parity error {err}"
    del g


def test_int8linear_module_and_memory():
    """The layer holds its int8 weight and scales only; layers share one forward
    workspace per device and stream, and the fused decode route needs none."""
    W, X = _small(24, 512, 128, seed=41)
    W2, _ = _small(24, 512, 128, seed=42)
    before = m8.shared_workspace_bytes()
    layer, layer2 = m8.Int8Linear(_dev(W), threshold=6.0), m8.Int8Linear(_dev(W2), threshold=6.0)
    Y = _host(layer(_dev(X).reshape(2, 12, 512)))
    Y2 = _host(layer2(_dev(X).reshape(2, 12, 512)))
    after = m8.shared_workspace_bytes()
    for Wi, Yi in ((W, Y), (W2, Y2)):
        Wq_ref, sW_ref = oracle.quantize_weight(Wi)
        st = oracle.linear(X, Wq_ref, sW_ref, 6.0)
        assert oracle.parity_error(Yi.reshape(24, 128), st.Y) <= Y_TOL
    assert layer.memory_bytes() == 128 * 512 + 4 * 128
    # T = 24 takes the GEMM route: one workspace for both layers, at most its size once
    need = m8.llmint8_workspace_bytes(24, 512, 128)
    assert need > 0 and after - before <= need
    # decode-sized calls (T <= gemv_max_rows) allocate nothing
    T = m8.llmint8_gemv_max_rows(512)
    assert m8.llmint8_workspace_bytes(T, 512, 128) == 0
    Yd = _host(layer(_dev(X[:T])))
    assert m8.shared_workspace_bytes() == after
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    assert oracle.parity_error(Yd, oracle.linear(X[:T], Wq_ref, sW_ref, 6.0).Y) <= Y_TOL


def test_decode_route_takes_no_workspace():
    """Through the C ABI: the fused decode route runs with a NULL workspace and gives
    the same bits as with one."""
    W, X = _small(4, 1024, 300, seed=43, n_out=5)
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Xd = _dev(X)
    lib = m8.load_library()
    Y0 = torch.empty((4, 300), dtype=torch.float16, device="cuda")
    st = lib.llmint8_linear(m8._ptr(Xd), 4, 1024, m8._ptr(Wq), m8._ptr(sW), 300, 6.0, m8._ptr(Y0),
                            None, 0, m8._stream(None, Xd.device))
    assert st == 0
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device="cuda")
    Y1 = m8.llmint8_linear(Xd, Wq, sW, 6.0, workspace=ws)
    assert np.array_equal(_host(Y0).view(np.uint16), _host(Y1).view(np.uint16))
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    assert oracle.parity_error(_host(Y0), oracle.linear(X, Wq_ref, sW_ref, 6.0).Y) <= Y_TOL


@pytest.mark.parametrize("tile", ["352x256", "256x256", "128x128"])
def test_outlier_chunks_past_the_workspace(tile):
    """|O| = 700 (22 chunks of 32 columns): a standard workspace holds the operands of
    the first 16 chunks and the epilogue forms the other 6 from X and Wq; a workspace
    large enough for all 22 must give the same bits, and both the oracle's values."""
    path = m8.LLMINT8_PATH_GEMM_TILES[tile]
    T, K, N = 300, 2048, 520
    rng = _rng(77)
    X = np.clip(workloads.random_fp16(rng, (T, K), 1.0).astype(np.float32), -5, 5).astype(np.float16)
    cols = np.sort(rng.choice(K, 700, replace=False))
    X[rng.integers(0, T, 700), cols] = np.float16(23.0)
    W = workloads.random_fp16(rng, (N, K), 0.05)
    err, c = run_case(f"700 outliers tile {tile}", W, X, 6.0, path)
    assert c == 700
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Xd = _dev(X)
    std = m8.llmint8_workspace_bytes_path(T, K, N, path)
    big = std + 6 * 2 * 32 * (T + N) + 4096
    ys = []
    for nbytes in (std, big):
        ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        out = m8.llmint8_linear_debug(Xd, Wq, sW, 6.0, path=path, workspace=ws, want_C=False)
        ys.append(_host(out["Y"]).view(np.uint16))
    assert np.array_equal(ys[0], ys[1]), "formed and held outlier chunks differ"


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

@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_workload(T):
    w = workloads.CONFIGS["decode"]
    W, X, _, _ = workloads.make(w, T=T)
    run_case(f"decode T={T}", W, X, w.threshold, GEMV, check_auto=True)
    run_case(f"decode T={T} gemm", W, X, w.threshold, GEMM)


def test_prefill_workload():
    w = workloads.CONFIGS["prefill"]
    W, X, _, _ = workloads.make(w)
    err, c = run_case("prefill", W, X, w.threshold, AUTO)
    assert c >= w.n_out


def test_large_workload():
    w = workloads.CONFIGS["large"]
    W, X, cols, zrows = workloads.make(w)
    err, c = run_case("large", W, X, w.threshold, AUTO)
    assert c >= w.n_out


@pytest.mark.parametrize("n_out", workloads.SWEEP_N_OUT)
def test_sweep_workload(n_out):
    w = workloads.CONFIGS["sweep"].with_(n_out=n_out)
    W, X, _, _ = workloads.make(w)
    for thr in workloads.SWEEP_THRESHOLDS:
        run_case(f"sweep n_out={n_out} thr={thr}", W, X, thr, AUTO)


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
