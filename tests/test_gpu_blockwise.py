"""GPU parity of the blockwise 8-bit codec, through the C ABI, against the oracle.

Codes, block maxima and dequantized values must be bit-exact, for fp16 and
fp32 tensors, every supported block size, ragged last blocks, zero blocks and
the full prefill weight.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu

BLOCKS = (64, 128, 256, 512, 1024, 2048, 4096)


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


def _check(x, block):
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, a = m8.llmint8_quantize_blockwise(xd, block)
    q_ref, a_ref = oracle.quantize_blockwise(x, block)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref), "codes differ"
    assert np.array_equal(a.cpu().numpy().view(np.uint32), a_ref.view(np.uint32)), "absmax differs"
    for dt, npdt in ((torch.float16, np.float16), (torch.float32, np.float32)):
        d = m8.llmint8_dequantize_blockwise(q, a, block, dtype=dt).cpu().numpy()
        d_ref = oracle.dequantize_blockwise(q_ref, a_ref, block, npdt)
        bits = np.uint16 if npdt == np.float16 else np.uint32
        assert np.array_equal(d.view(bits), d_ref.view(bits)), f"dequantized {npdt} differs"


def _data(seed, n, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * 0.5
    x[rng.random(n) < 0.001] *= 200.0          # isolated large values
    if n >= 3 * 4096:
        x[4096:8192] = 0.0                       # zero blocks
    return x.astype(dtype)


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("n", [16, 4096 + 16, 100000, 1 << 20])
def test_blockwise_bit_exact(block, dtype, n):
    _say(f"blockwise block={block} dtype={np.dtype(dtype).name} n={n}")
    _check(_data(block + n, n, dtype), block)


def test_blockwise_prefill_weight_and_state():
    w = workloads.CONFIGS["prefill"]
    W = workloads.make_weight(workloads.rng_for(w.seed, 0), w.N, w.K, w.sigma).reshape(-1)
    for block in (64, 4096):
        _say(f"blockwise prefill weight n={W.size} block={block}")
        _check(W, block)
    S = workloads.make_state(w.seed, 1 << 24)
    _say(f"blockwise optimizer-state tensor n={S.size}")
    _check(S, 2048)


def test_blockwise_edge_cases():
    _say("blockwise edge cases")
    empty = torch.empty((0,), dtype=torch.float16, device="cuda")
    q, a = m8.llmint8_quantize_blockwise(empty, 64)
    assert q.numel() == 0 and a.numel() == 0
    x = torch.zeros((40,), dtype=torch.float16, device="cuda")
    with pytest.raises(m8.Llmint8Error) as e:                # n % 16 != 0
        m8.llmint8_quantize_blockwise(x, 64)
    assert e.value.status == -2
    x = torch.zeros((4096,), dtype=torch.float16, device="cuda")
    for bad in (96, 32, 8192):
        with pytest.raises(m8.Llmint8Error) as e:
            m8.llmint8_quantize_blockwise(x, bad)
        assert e.value.status == -2
    q, a = m8.llmint8_quantize_blockwise(x, 64)               # all-zero tensor
    assert not torch.any(q) and not torch.any(a)
    assert not torch.any(m8.llmint8_dequantize_blockwise(q, a, 64))


@pytest.mark.parametrize("i", range(30))
def test_blockwise_random_sweep(i):
    """Seeded random lengths (multiples of 16 up to 3 M), block sizes, input types
    and value scales (down to subnormal fp16 and up to 1e4): codes, maxima and
    both dequantized types bit-exact."""
    rng = np.random.default_rng(5000 + i)
    n = 16 * int(rng.integers(1, 200000))
    block = int(rng.choice(BLOCKS))
    dtype = np.float16 if rng.random() < 0.5 else np.float32
    scale = float(10.0 ** rng.uniform(-6, 4))
    x = rng.standard_normal(n) * scale
    x[rng.random(n) < 0.01] = 0.0
    _say(f"blockwise sweep {i}: n={n} block={block} dtype={np.dtype(dtype).name} scale={scale:.3g}")
    with np.errstate(over="ignore"):
        x = x.astype(dtype)
    _check(x, block)
