"""GPU parity of the 4-bit weight path (NF4 / FP4), through the C ABI, against the oracle.

Bar: packed codes, block maxima and dequantized 16-bit weights bit-exact; Y of
the 4-bit linear within the 16-bit output bar of ``parity_util`` (the kernel
sums fp32 products in its own order, the oracle sums exactly).

Sources (page title, section): "bitsandbytes" (glossary), "What it provides"
(FP4 and NF4, blockwise scaling, 16-bit compute with the weight dequantized
per operation); "Hugging Face
Quantization with bitsandbytes ...", section 4.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from parity_util import check_y

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu


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
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _as(dtype, a):
    return workloads.as_bf16_input(a) if dtype == "bf16" else a


def _tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def codec_case(name, w16, block, quant_type, dtype):
    """Quantize and dequantize on the GPU; both bit-exact against the oracle."""
    n = w16.size
    _say(f"{name}: {quant_type} {dtype} n={n} block={block}")
    packed, a = m8.llmint8_quantize_4bit(_dev(w16), block, quant_type)
    p_ref, a_ref = oracle.quantize_4bit(w16, block, quant_type, dtype)
    assert np.array_equal(_host(packed), p_ref), "codes differ"
    assert np.array_equal(_host(a).view(np.uint32), a_ref.view(np.uint32)), "absmax differs"
    d = m8.llmint8_dequantize_4bit(packed, a, block, quant_type, dtype=_tdtype(dtype))
    d_ref = oracle.dequantize_4bit(p_ref, a_ref, block, quant_type, n, dtype)
    assert np.array_equal(_host(d).view(np.uint16), np.ascontiguousarray(d_ref).view(np.uint16)), \
        "dequantized values differ"
    return packed, a


def linear_case(name, W, X, block, quant_type, dtype, bias=None, rows=None):
    """4-bit linear on the GPU against the oracle (optionally on a sample of weight rows)."""
    T, K = X.shape
    N = W.shape[0]
    _say(f"{name}: {quant_type} {dtype} T={T} K={K} N={N} block={block} bias={bias is not None}")
    packed, a = m8.llmint8_quantize_4bit(_dev(W), block, quant_type)
    Y = m8.llmint8_linear_4bit(_dev(X), packed, a, N, block, quant_type,
                               bias=None if bias is None else _dev(bias))
    Yh = _host(Y)
    if rows is None:
        p_ref, a_ref = oracle.quantize_4bit(W, block, quant_type, dtype)
        ref = oracle.linear_4bit(X, p_ref, a_ref, block, quant_type, N, dtype, bias)
        got = Yh
    else:
        # rows of the weight are independent: quantize and multiply the sampled rows only
        assert K % block == 0
        Ws = np.ascontiguousarray(W[rows])
        p_ref, a_ref = oracle.quantize_4bit(Ws, block, quant_type, dtype)
        ph = _host(packed).reshape(N, K // 2)[rows]
        ah = _host(a).reshape(N, K // block)[rows]
        assert np.array_equal(ph.reshape(-1), p_ref), "sampled codes differ"
        assert np.array_equal(ah.reshape(-1).view(np.uint32), a_ref.view(np.uint32))
        ref = oracle.linear_4bit(X, p_ref, a_ref, block, quant_type, len(rows), dtype,
                                 None if bias is None else bias[rows])
        got = Yh[:, rows]
    if dtype == "bf16":
        return check_y(np.ascontiguousarray(got).view(np.uint16), ref, "bf16")
    return check_y(got, ref, "f16")


def _weights(seed, N, K, sigma=0.02):
    return workloads.make_weight(workloads.rng_for(seed, 0), N, K, sigma)


def _acts(seed, T, K):
    return workloads.random_fp16(workloads.rng_for(seed, 1), (T, K))


# --------------------------------------------------------------------------- codec

@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("block", [64, 128, 256, 1024, 4096])
def test_codec_ragged_and_zero_blocks(quant_type, dtype, block):
    for n in (16, 4112, 100000):
        w = (np.random.default_rng(n + block).standard_normal(n) * 0.05).astype(np.float16)
        w[n // 3: n // 3 + 3 * block] = 0                      # at least two zero blocks
        w[n // 2] = np.float16(30.0)                            # an isolated large value
        codec_case(f"codec n={n}", _as(dtype, w), block, quant_type, dtype)


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_codec_level_values_and_midpoints(quant_type):
    """Blocks whose maximum is 1, holding every level and the fp16-exact midpoints."""
    book = oracle.code_book(quant_type)
    _, mids = oracle.quantize_levels(quant_type)
    vals = np.concatenate([book.astype(np.float16).astype(np.float32),
                           mids[mids.astype(np.float16).astype(np.float32) == mids],
                           np.nextafter(mids, np.float32(1)), np.nextafter(mids, np.float32(-1))])
    w = np.zeros(64 * 4, np.float32)
    w[: vals.size] = vals
    w[::64] = 1.0
    codec_case("levels", w.astype(np.float16), 64, quant_type, "f16")


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_codec_decode_weight(quant_type, dtype):
    W = _weights(2, 4096, 4096)
    codec_case("decode weight", _as(dtype, W), 64, quant_type, dtype)


# --------------------------------------------------------------------------- linear

@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N,block", [(1, 128, 1, 64), (3, 384, 17, 64), (16, 512, 200, 128),
                                         (17, 256, 33, 64), (40, 1024, 48, 256),
                                         (5, 4096, 100, 4096), (2, 640, 64, 64)])
def test_linear_small(quant_type, dtype, T, K, N, block):
    W, X = _weights(T + K, N, K, 0.05), _acts(T + K + N, T, K)
    b = workloads.make_bias(N, N, bf16=dtype == "bf16")
    linear_case("small", _as(dtype, W), _as(dtype, X), block, quant_type, dtype)
    linear_case("small bias", _as(dtype, W), _as(dtype, X), block, quant_type, dtype, bias=b)


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T", [1, 4, 8])
def test_linear_decode_workload(quant_type, dtype, T):
    w = workloads.CONFIGS["decode"]
    W, X, _, _ = workloads.make(w, T=T)
    b = workloads.make_bias(w.seed, w.N, bf16=dtype == "bf16")
    linear_case("decode", _as(dtype, W), _as(dtype, X), 64, quant_type, dtype, bias=b)


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,K,N,block", [(20, 384, 8200, 64), (4, 1152, 16408, 128),
                                         (17, 2048, 8232, 64), (17, 8320, 8200, 64)])
def test_linear_two_row_blocks(quant_type, dtype, T, K, N, block):
    """Shapes that take 32 weight rows per workgroup on a 256-CU device (T >= 4,
    ceil(N/32) x ceil(T/16) >= 512): ragged N (a last workgroup with one row
    block partly or wholly past N), T past 16, odd step counts and steps left
    to some wavefronts only, with bias; every output against the oracle."""
    W, X = _weights(T + K + N, N, K, 0.05), _acts(T + K + N + 1, T, K)
    b = workloads.make_bias(N, N, bf16=dtype == "bf16")
    linear_case("two row blocks", _as(dtype, W), _as(dtype, X), block, quant_type, dtype, bias=b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_linear_large_layer_sampled_rows(dtype):
    w = workloads.CONFIGS["large"]
    W = _weights(w.seed, w.N, w.K, w.sigma)
    X = workloads.make(w, T=8, with_weight=False)[1]
    rows = np.unique(np.concatenate([np.sort(np.random.default_rng(5).choice(w.N, 96, replace=False)),
                                     [0, w.N - 1]]))
    b = workloads.make_bias(w.seed, w.N, bf16=dtype == "bf16")
    linear_case("large layer", _as(dtype, W), _as(dtype, X), 64, "nf4", dtype, bias=b, rows=rows)


def test_repeat_calls_bit_identical_and_module():
    W, X = _weights(7, 300, 1024), _acts(8, 6, 1024)
    Wd, Xd = _dev(W), _dev(X)
    packed, a = m8.llmint8_quantize_4bit(Wd, 64, "nf4")
    ys = [_host(m8.llmint8_linear_4bit(Xd, packed, a, 300, 64, "nf4")).view(np.uint16)
          for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    layer = m8.Linear4bit(Wd, bias=_dev(workloads.make_bias(9, 300)), block=64)
    Y = _host(layer(Xd.reshape(2, 3, 1024))).reshape(6, 300)
    p_ref, a_ref = oracle.quantize_4bit(W, 64, "nf4")
    ref = oracle.linear_4bit(X, p_ref, a_ref, 64, "nf4", 300, "f16", workloads.make_bias(9, 300))
    check_y(Y, ref, "f16")
    assert layer.memory_bytes() == 300 * 1024 // 2 + 4 * (300 * 1024 // 64) + 2 * 300


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_linear_long_rows(quant_type):
    """K = 65536: each of the 16 wavefronts of a row block walks 32 steps."""
    W, X = _weights(67, 40, 65536, 0.02), _acts(68, 3, 65536)
    linear_case("K=65536", W, X, 256, quant_type, "f16", bias=workloads.make_bias(69, 40))


@pytest.mark.parametrize("i", range(40))
def test_linear_random_sweep(i):
    """Seeded random decode shapes (T up to 40, K up to 5120, N up to 600), block
    sizes, both code books, both 16-bit types, with and without bias: codes,
    maxima and dequantized weights bit-exact, Y within the bar of its type."""
    rng = np.random.default_rng(6000 + i)
    T = int(rng.integers(1, 41))
    K = 128 * int(rng.integers(1, 41))
    N = int(rng.integers(1, 601))
    block = int(rng.choice([b for b in (64, 128, 256, 512, 1024, 2048, 4096) if b <= max(64, K)]))
    quant_type = str(rng.choice(["nf4", "fp4"]))
    dtype = "bf16" if rng.random() < 0.5 else "f16"
    W, X = _weights(6100 + i, N, K, 0.05), _acts(6200 + i, T, K)
    b = workloads.make_bias(6300 + i, N, bf16=dtype == "bf16") if rng.random() < 0.5 else None
    codec_case(f"sweep {i} codec", _as(dtype, W), block, quant_type, dtype)
    linear_case(f"sweep {i}", _as(dtype, W), _as(dtype, X), block, quant_type, dtype, bias=b)
