"""GPU parity of the bf16 forward and the fused bias, through the C ABI, against the oracle.

Bar: outlier set, int8 codes, row/column statistics and int32 accumulators
bit-exact, as for fp16. Y: with fp16 output, max-abs-relative error <= 1e-3; with
bf16 output, which has 8 significant bits, the kernel's fp32 sum and the
oracle's exact one may straddle a rounding boundary, so every element must be
the oracle's bf16 value or one of its two neighbours (or within 2**-16 of the
largest |Y|, the fp32 arithmetic's own slack where terms cancel), at least 99%
of the elements must be bit-identical, and the max-abs-relative error must stay
<= 2**-7 (one bf16 step at the largest |Y|).

Sources (page title, section): "Hugging Face Quantization with bitsandbytes ...",
section 5 (bfloat16 as the compute type); "bitsandbytes: GPU-Accelerated
Inference ..." (Linear8bitLt replaces a linear layer, which has a bias).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity_util import check_y

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu

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
    """numpy fp16 array, or uint16 bf16 bit patterns, -> CUDA tensor of that type."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def quantize_weight_checked(W, dtype):
    Wq_ref, sW_ref = oracle.quantize_weight(W, dtype)
    Wq, sW = m8.llmint8_quantize_weight_ex(_dev(W))
    assert np.array_equal(_host(Wq), Wq_ref), "Wq differs"
    assert np.array_equal(_host(sW).view(np.uint32), sW_ref.view(np.uint32)), "sW differs"
    return Wq, sW, Wq_ref, sW_ref


def run_case(name, W, X, thr, path, dtype, bias=None, rows=None, check_plain=True):
    """One forward on the GPU through the _ex entry points, every stage against the oracle."""
    T, K = X.shape
    N = W.shape[0]
    _say(f"{name}: {dtype} T={T} K={K} N={N} thr={thr} path={path} bias={bias is not None}")
    Wq, sW, Wq_ref, sW_ref = quantize_weight_checked(W, dtype)
    Xd = _dev(X)
    bd = None if bias is None else _dev(bias)
    out = m8.llmint8_linear_debug_ex(Xd, Wq, sW, thr, bias=bd, path=path, want_C=True)
    st = oracle.linear(X, Wq_ref, sW_ref, thr, rows=rows, dtype=dtype, bias=bias)
    count = int(_host(out["count"])[0])
    assert count == st.count, (count, st.count)
    assert np.array_equal(_host(out["bitmap"]).view(np.uint32), st.bitmap)
    assert np.array_equal(_host(out["idx"])[:count], st.idx)
    assert np.array_equal(_host(out["Xq"]), st.Xq), "Xq differs"
    assert np.array_equal(_host(out["aX"]).view(np.uint32), st.aX.view(np.uint32)), "aX differs"
    sel = slice(None) if rows is None else rows
    assert np.array_equal(_host(out["C"])[sel], st.C), "C differs"
    Y = _host(out["Y"])
    err = check_y(_bits16(Y[sel]) if dtype == "bf16" else Y[sel],
                  _bits16(st.Y) if dtype == "bf16" else st.Y, dtype)
    if check_plain:
        Y2 = m8.llmint8_linear_ex(Xd, Wq, sW, thr, bias=bd)
        assert np.array_equal(_bits16(_host(Y2)), _bits16(Y)), "plain call differs"
    return err, count


def _small(T, K, N, seed, n_out=3, lo=20.0, hi=60.0, sigma=0.05):
    w = workloads.Workload("edge", T=T, K=K, N=N, sigma=sigma, n_out=min(n_out, K), lo=lo, hi=hi,
                           threshold=6.0, seed=seed)
    W, X, _, _ = workloads.make(w)
    return W, X


def _as(dtype, *arrays):
    if dtype == "bf16":
        return tuple(workloads.as_bf16_input(a) for a in arrays)
    return arrays


def _bias(seed, N, dtype, on=True):
    return workloads.make_bias(seed, N, bf16=dtype == "bf16") if on else None


# --------------------------------------------------------------------------- small, full compare

@pytest.mark.parametrize("N,K", [(200, 256), (17, 1040), (1000, 272), (64, 8192), (3, 48)])
def test_bf16_weight_quantization(N, K):
    _say(f"bf16 weight quantization N={N} K={K}")
    W = workloads.as_bf16_input(workloads.random_fp16(np.random.default_rng(N + K), (N, K), 0.05))
    W[0, : min(K, 5)] = 0x3F80                        # 1.0 ties in one row
    if N > 2:
        W[2] = 0                                      # an all-zero row
    quantize_weight_checked(W, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [1, 3, 9, 16, 33, 130, 300])
def test_ragged_rows_with_bias(dtype, T):
    W, X = _as(dtype, *_small(T, 256, 200, seed=300 + T))
    for path in ([GEMM, GEMV] if T <= 16 else [GEMM]):
        run_case(f"ragged T={T}", W, X, 6.0, path, dtype, bias=_bias(T, 200, dtype))


@pytest.mark.parametrize("T", [1, 5, 130])
def test_bf16_without_bias(T):
    W, X = _as("bf16", *_small(T, 512, 136, seed=400 + T))
    for path in ([GEMM, GEMV] if T <= 16 else [GEMM]):
        run_case(f"bf16 no bias T={T}", W, X, 6.0, path, "bf16")


@pytest.mark.parametrize("K,N", [(16, 1), (48, 3), (1040, 17), (4112, 250), (272, 1000), (8192, 64)])
def test_bf16_ragged_k_and_n(K, N):
    W, X = _as("bf16", *_small(37, K, N, seed=K + N + 1))
    b = _bias(K, N, "bf16")
    run_case(f"bf16 ragged K={K} N={N}", W, X, 6.0, GEMM, "bf16", bias=b)
    run_case(f"bf16 ragged K={K} N={N} gemv", W, X[:5], 6.0, GEMV, "bf16", bias=b)


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_bf16_threshold_edges(path):
    W, X = _as("bf16", *_small(12, 512, 96, seed=8))
    run_case("bf16 thr=inf", W, X, math.inf, path, "bf16", bias=_bias(1, 96, "bf16"))
    X2 = workloads.as_bf16_input(np.clip(workloads.random_fp16(np.random.default_rng(2), (12, 512)),
                                         -5, 5))
    _, c = run_case("bf16 no outlier", W, X2, 6.0, path, "bf16")
    assert c == 0
    X3 = workloads.as_bf16_input(np.clip(workloads.random_fp16(np.random.default_rng(3), (11, 512)),
                                         -5.5, 5.5))
    X3[2, 17] = 0x40C0          # 6.0 exactly: an outlier
    X3[4, 33] = 0xC0C0          # -6.0
    X3[5, 70] = 0x40BF          # 5.96875, the bf16 just below 6: not an outlier
    X3[7] = 0                   # an all-zero row
    X3[8, :] = 0x4020           # 2.5 everywhere: rounding ties after scaling
    _, c = run_case("bf16 ties", W, X3, 6.0, path, "bf16", bias=_bias(2, 96, "bf16"))
    assert c == 2


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_bf16_every_column_outlier(path):
    rng = np.random.default_rng(4)
    X = workloads.random_fp16(rng, (9, 96), 2.0)
    X[X == 0] = np.float16(0.5)
    W = workloads.random_fp16(rng, (40, 96), 0.05)
    W, X = _as("bf16", W, X)
    _, c = run_case("bf16 all columns", W, X, 1e-3, path, "bf16", bias=_bias(3, 40, "bf16"))
    assert c == 96


def test_bf16_many_outlier_chunks():
    W, X = _as("bf16", *_small(70, 1024, 300, seed=22, n_out=100))
    b = _bias(4, 300, "bf16")
    _, c = run_case("bf16 100 outliers", W, X, 6.0, GEMM, "bf16", bias=b)
    assert c >= 100
    run_case("bf16 100 outliers gemv", W, X[:9], 6.0, GEMV, "bf16", bias=b)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("tile", sorted(m8.LLMINT8_PATH_GEMM_TILES))
def test_every_gemm_tile_with_bias(dtype, tile):
    path = m8.LLMINT8_PATH_GEMM_TILES[tile]
    for (T, K, N, n_out, seed) in ((300, 1040, 1000, 3, 31), (70, 1024, 706, 100, 32)):
        W, X = _as(dtype, *_small(T, K, N, seed=seed, n_out=n_out))
        run_case(f"tile {tile}", W, X, 6.0, path, dtype, bias=_bias(seed, N, dtype))


@pytest.mark.parametrize("path", [GEMM, GEMV])
def test_fp16_ex_without_bias_matches_the_plain_entry(path):
    W, X = _small(7, 1024, 264, seed=61)
    Wq, sW = m8.llmint8_quantize_weight(_dev(W))
    Wq2, sW2 = m8.llmint8_quantize_weight_ex(_dev(W))
    assert torch.equal(Wq, Wq2) and torch.equal(sW.view(torch.int32), sW2.view(torch.int32))
    Xd = _dev(X)
    Y1 = m8.llmint8_linear_debug(Xd, Wq, sW, 6.0, path=path)["Y"]
    Y2 = m8.llmint8_linear_debug_ex(Xd, Wq, sW, 6.0, path=path)["Y"]
    assert np.array_equal(_bits16(_host(Y1)), _bits16(_host(Y2)))


def test_int8linear_bf16_with_bias():
    W, X = _as("bf16", *_small(24, 512, 128, seed=42))
    b = _bias(5, 128, "bf16")
    _say("Int8Linear bf16 + bias")
    layer = m8.Int8Linear(_dev(W), threshold=6.0, bias=_dev(b))
    Y = _host(layer(_dev(X).reshape(2, 12, 512)))
    Wq_ref, sW_ref = oracle.quantize_weight(W, "bf16")
    st = oracle.linear(X, Wq_ref, sW_ref, 6.0, dtype="bf16", bias=b)
    check_y(_bits16(Y.reshape(24, 128)), _bits16(st.Y), "bf16")
    assert layer.memory_bytes() == 128 * 512 + 4 * 128 + 2 * 128


# --------------------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("T", [1, 8])
def test_bf16_decode_workload(T):
    w = workloads.CONFIGS["decode"]
    W, X = _as("bf16", *workloads.make(w, T=T)[:2])
    b = _bias(w.seed, w.N, "bf16")
    run_case(f"bf16 decode T={T}", W, X, w.threshold, GEMV, "bf16", bias=b)
    run_case(f"bf16 decode T={T} gemm", W, X, w.threshold, GEMM, "bf16", bias=b, check_plain=False)


def test_bf16_prefill_workload():
    w = workloads.CONFIGS["prefill"]
    W, X = _as("bf16", *workloads.make(w)[:2])
    b = _bias(w.seed, w.N, "bf16")
    _, c = run_case("bf16 prefill", W, X, w.threshold, AUTO, "bf16", bias=b)
    assert c >= w.n_out


def test_timed_ex_records_kernel_events():
    W, X = _as("bf16", *_small(256, 1024, 512, seed=52))
    b = _bias(6, 512, "bf16")
    _say("timed_ex bf16 + bias")
    Wq, sW = m8.llmint8_quantize_weight_ex(_dev(W))
    Xd, bd = _dev(X), _dev(b)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    ws = torch.empty((m8.llmint8_workspace_bytes(256, 1024, 512),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda")
    nk = m8.llmint8_linear_timed_ex(Xd, Wq, sW, 6.0, Y, ws, ev, bias=bd, path=GEMM)
    torch.cuda.synchronize()
    assert nk == 3
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(3))
    Y2 = m8.llmint8_linear_ex(Xd, Wq, sW, 6.0, bias=bd, workspace=ws)
    assert np.array_equal(_host(Y), _host(Y2))
