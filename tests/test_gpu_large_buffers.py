"""GPU regression tests on buffers larger than 2 GiB, within the C ABI's limits.

The kernels read ragged edges through buffer loads whose "reads as zero"
offset is 2^31; each resource they build must span at most 2^31 bytes for that
offset to lie outside it (checked for every admitted shape on the CPU by
tests/test_ranges.py). These cases run the kernels where a single resource over
the whole tensor would be larger than 2 GiB, with a large value planted at the
byte offset 2^31 of the input, where an in-range "zero" read would land:
  * the int8 forward at T = 131200, K = 8192 (X is 2.15 GB): outlier set, row
    statistics and int8 codes over all rows bit-exact (the oracle runs over row
    chunks; the outlier set is a union over rows), C and Y on sampled rows;
  * the blockwise 8-bit codec on an fp32 tensor of 2^29 + 48 elements (2.15 GB)
    with a ragged last block: codes, block maxima and dequantized values
    bit-exact over the whole tensor, blocks of 64 and 4096;
  * the 4-bit codec on 2^30 + 48 fp16 elements: codes and block maxima of the
    blocks around the 2 GiB offset and of the ragged last block bit-exact.
Page: "Hugging Face Quantization with bitsandbytes ...", sections 2 and 3 (the
outlier set is decided over all rows of the call); "bitsandbytes" glossary,
"What it provides" (blockwise scaling).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


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
    torch.cuda.empty_cache()


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_int8_forward_with_activations_over_2gib():
    T, K, N, thr = 131200, 8192, 64, 6.0
    assert T * K * 2 > 2 ** 31 and T * K < 2 ** 31
    _say(f"int8 forward T={T} K={K} N={N}: X {T * K * 2 / 2**30:.2f} GiB")
    rng = np.random.default_rng(2024)
    X = workloads.random_fp16_large(rng, (T, K), 1.0)
    np.clip(X, np.float16(-5.0), np.float16(5.0), out=X)
    # flat element 2^30 (byte 2^31) is row 131072, column 0: a large value there
    # must count for its own column only
    X[131072, 3] = np.float16(50.0)
    X[17, 4000] = np.float16(-30.0)
    X[T - 1, 8191] = np.float16(7.5)
    W = workloads.random_fp16(rng, (N, K), 0.02)
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    Wq, sW = m8.llmint8_quantize_weight(torch.from_numpy(W).cuda())
    Xd = torch.from_numpy(X).cuda()
    out = m8.llmint8_linear_debug(Xd, Wq, sW, thr, path=m8.LLMINT8_PATH_GEMM, want_C=True)
    del Xd
    count = int(_host(out["count"])[0])
    bitmap = _host(out["bitmap"]).view(np.uint32)
    idx = _host(out["idx"])[:count]
    aX = _host(out["aX"])
    Xq_gpu = _host(out["Xq"])
    C = _host(out["C"])
    Y = _host(out["Y"])
    del out
    # the oracle over row chunks: the outlier set is the union of the chunks' sets,
    # the row statistics and codes are per row
    step = 8192
    mask = np.zeros(K, bool)
    for r0 in range(0, T, step):
        mask |= oracle.outlier_columns(X[r0:r0 + step], thr)
    ref_idx = np.flatnonzero(mask).astype(np.int32)
    assert count == ref_idx.size == 3, (count, ref_idx)
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(bitmap, oracle.pack_bitmap(mask))
    aX_ref = np.empty(T, np.float32)
    for r0 in range(0, T, step):
        q, a = oracle.quantize_activations(X[r0:r0 + step], mask)
        aX_ref[r0:r0 + step] = a
        assert np.array_equal(Xq_gpu[r0:r0 + step], q), f"Xq differs in rows {r0}.."
    assert np.array_equal(aX.view(np.uint32), aX_ref.view(np.uint32)), "aX differs"
    rows = np.unique(np.concatenate([np.sort(rng.choice(T, 40, replace=False)),
                                     [0, 17, 131071, 131072, 131073, T - 2, T - 1],
                                     np.arange(16399, 16401), np.arange(T - 70, T - 60)]))
    Xq_rows = Xq_gpu[rows]
    C_ref = oracle.int8_matmul(Xq_rows, Wq_ref)
    assert np.array_equal(C[rows], C_ref), "C differs"
    Xo, Wd = oracle.outlier_operands(X[rows], Wq_ref, sW_ref, ref_idx)
    Y_ref = oracle.output(C_ref, aX_ref[rows], sW_ref, Xo, Wd)
    err = oracle.parity_error(Y[rows], Y_ref)
    assert err <= 1e-3, err


@pytest.mark.parametrize("block", [64, 4096])
def test_blockwise_fp32_over_2gib_ragged(block):
    n = 2 ** 29 + 48
    assert n * 4 > 2 ** 31
    _say(f"blockwise fp32 n={n} block={block}")
    rng = np.random.default_rng(7)
    x = (workloads.random_fp16_large(rng, (n,), 1e-3)).astype(np.float32)
    x[2 ** 29] = np.float32(1000.0)        # byte 2^31: the first element of the ragged last block
    x[2 ** 29 - 5] = np.float32(-250.0)
    xd = torch.from_numpy(x).cuda()
    q, a = m8.llmint8_quantize_blockwise(xd, block)
    deq = m8.llmint8_dequantize_blockwise(q, a, block, dtype=torch.float32)
    del xd
    qh, ah, dh = _host(q), _host(a), _host(deq)
    del q, a, deq
    q_ref, a_ref = oracle.quantize_blockwise(x, block)
    assert np.array_equal(ah.view(np.uint32), a_ref.view(np.uint32)), "absmax differs"
    assert np.array_equal(qh, q_ref), "codes differ"
    d_ref = oracle.dequantize_blockwise(q_ref, a_ref, block, np.float32)
    assert np.array_equal(dh.view(np.uint32), d_ref.view(np.uint32)), "dequantized values differ"


def test_4bit_codes_over_2gib():
    n, block = 2 ** 30 + 48, 64
    assert n * 2 > 2 ** 31
    _say(f"4-bit nf4 n={n} block={block}")
    rng = np.random.default_rng(8)
    w = workloads.random_fp16_large(rng, (n,), 0.02)
    w[2 ** 30] = np.float16(3.0)           # byte 2^31: the first element of the ragged last block
    w[2 ** 30 - 1] = np.float16(-2.0)
    wd = torch.from_numpy(w).cuda()
    packed, a = m8.llmint8_quantize_4bit(wd, block, "nf4")
    del wd
    ph, ah = _host(packed), _host(a)
    nb = ah.size
    # blocks are independent: check those around the 2 GiB offset, the ragged last
    # block and a seeded sample, each against the oracle on its own elements
    blocks = np.unique(np.concatenate([np.arange(nb - 40, nb), np.arange(2 ** 24 - 40, 2 ** 24),
                                       rng.choice(nb, 200, replace=False)]))
    for b in blocks:
        e0, e1 = b * block, min(n, (b + 1) * block)
        p_ref, a_ref = oracle.quantize_4bit(w[e0:e1], block, "nf4")
        assert ah[b].view(np.uint32) == a_ref[0].view(np.uint32), f"absmax of block {b}"
        assert np.array_equal(ph[e0 // 2:(e1 + 1) // 2], p_ref), f"codes of block {b}"
