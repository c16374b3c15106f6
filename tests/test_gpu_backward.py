"""GPU parity of the input gradient through the frozen int8 layer.

Called through the C ABI and compared with the CPU oracle on the same seeded
inputs: the dequantized, transposed weight bit-exact; dX within
max-abs-relative 1e-3 (fp32 summation order is not pinned). Small and ragged
shapes compare every element; the prefill-sized backward compares a seeded
sample of rows. The input gradient forms the dequantized weight on the fly,
inside its GEMM; with a one-hot output gradient (dY[t, n] = 1 for one n per
row) each row of dX is a row of that operand exactly (one product by 1, an
exact fp32 sum and an exact rounding), which checks the on-the-fly
dequantization bit for bit.
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

DX_TOL = 1e-3


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


def _weights(seed, N, K, sigma=0.02):
    W = workloads.make_weight(workloads.rng_for(seed, 0), N, K, sigma)
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    return _dev(Wq_ref), _dev(sW_ref), Wq_ref, sW_ref


@pytest.mark.parametrize("N,K", [(64, 128), (200, 336), (8, 16), (1000, 1040)])
def test_dequantize_transposed_bit_exact(N, K):
    _say(f"dequantize_weight_t N={N} K={K}")
    Wq, sW, Wq_ref, sW_ref = _weights(21, N, K)
    WdT = _host(m8.llmint8_dequantize_weight_t(Wq, sW))
    ref = oracle.dequantize_weight(Wq_ref, sW_ref).T
    assert np.array_equal(WdT.view(np.uint16), ref.view(np.uint16))


def test_dequantize_transposed_prefill_weight_bit_exact():
    w = workloads.CONFIGS["prefill"]
    _say(f"dequantize_weight_t N={w.N} K={w.K}")
    W = workloads.make_weight(workloads.rng_for(w.seed, 0), w.N, w.K, w.sigma)
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    WdT = _host(m8.llmint8_dequantize_weight_t(_dev(Wq_ref), _dev(sW_ref)))
    ref = oracle.dequantize_weight(Wq_ref, sW_ref).T
    assert np.array_equal(WdT.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("N,K,dtype", [(520, 272, "f16"), (1000, 1040, "f16"), (72, 16, "f16"),
                                       (2056, 4112, "bf16"), (11008, 4096, "f16")])
def test_on_the_fly_dequantization_bit_exact(N, K, dtype):
    """dY one-hot over a permutation of the weight rows: dX row t = Wdeq row perm[t]."""
    _say(f"backward one-hot N={N} K={K} {dtype}")
    Wq, sW, Wq_ref, sW_ref = _weights(27, N, K)
    rng = np.random.default_rng(N + K)
    T = min(N, 2048)
    perm = rng.permutation(N)[:T]
    one = np.uint16(0x3C00 if dtype == "f16" else 0x3F80)      # 1.0 in fp16 / bf16
    dY = np.zeros((T, N), np.uint16)
    dY[np.arange(T), perm] = one
    dYd = _dev(dY).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    dX = _host(m8.llmint8_linear_backward_input_ex(dYd, Wq, sW).view(torch.int16)).view(np.uint16)
    ref = oracle.dequantize_weight(Wq_ref, sW_ref, dtype)
    ref = ref.view(np.uint16) if ref.dtype != np.uint16 else ref
    assert np.array_equal(dX, ref[perm]), "on-the-fly dequantized operand differs"


@pytest.mark.parametrize("T,K,N", [(16, 1024, 1024), (37, 336, 200), (300, 512, 264),
                                   (1, 4096, 4096), (257, 144, 520), (5, 16, 8)])
def test_backward_input_parity(T, K, N):
    _say(f"backward_input T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = _weights(22, N, K)
    dY = workloads.make_output_grad(22, T, N)
    dX = _host(m8.llmint8_linear_backward_input(_dev(dY), Wq, sW))
    ref = oracle.linear_backward_input(dY, Wq_ref, sW_ref)
    assert np.all(np.isfinite(dX.astype(np.float32)))
    err = oracle.parity_error(dX, ref)
    assert err <= DX_TOL, err


@pytest.mark.parametrize("cfg", ["prefill", "large"])
def test_backward_input_full_size_sampled_rows(cfg):
    """Backward of the workload's layer at full size (the launch the benchmark
    times); a seeded sample of 24 rows of dX is checked against the oracle."""
    w = workloads.CONFIGS[cfg]
    _say(f"backward_input {cfg} T={w.T} K={w.K} N={w.N}")
    W = workloads.make_weight(workloads.rng_for(w.seed, 0), w.N, w.K, w.sigma)
    Wq_ref, sW_ref = oracle.quantize_weight(W)
    del W
    dY = workloads.make_output_grad(w.seed, w.T, w.N)
    dX = _host(m8.llmint8_linear_backward_input(_dev(dY), _dev(Wq_ref), _dev(sW_ref)))
    rows = np.sort(np.random.default_rng(w.seed).choice(w.T, size=24, replace=False))
    rows = np.unique(np.concatenate([rows, [0, w.T - 1]]))
    ref = oracle.linear_backward_input(dY[rows], Wq_ref, sW_ref)
    assert np.all(np.isfinite(dX.astype(np.float32)))
    err = oracle.parity_error(dX[rows], ref)
    assert err <= DX_TOL, err


def test_backward_input_edge_cases():
    _say("backward_input edge cases")
    Wq, sW, _, _ = _weights(23, 64, 128)
    empty = m8.llmint8_linear_backward_input(_dev(np.zeros((0, 64), np.float16)), Wq, sW)
    assert tuple(empty.shape) == (0, 128)
    # N % 8 != 0 is rejected before anything runs
    Wq2, sW2, _, _ = _weights(23, 60, 128)
    with pytest.raises(m8.Llmint8Error) as e:
        m8.llmint8_linear_backward_input(_dev(np.zeros((4, 60), np.float16)), Wq2, sW2)
    assert e.value.status == -2
    # no workspace is needed; one given is ignored
    small = torch.empty((256,), dtype=torch.uint8, device="cuda")
    dY4 = _dev(workloads.make_output_grad(25, 4, 64))
    a = _host(m8.llmint8_linear_backward_input(dY4, Wq, sW, workspace=small)).view(np.uint16)
    b = _host(m8.llmint8_linear_backward_input(dY4, Wq, sW)).view(np.uint16)
    assert np.array_equal(a, b)
    # a zero gradient gives an exact zero
    dX = _host(m8.llmint8_linear_backward_input(_dev(np.zeros((3, 64), np.float16)), Wq, sW))
    assert not np.any(dX.astype(np.float32))


def test_int8linear_autograd_uses_the_kernels():
    """Int8Linear in autograd: X.grad is the library's input gradient, bit for bit."""
    _say("Int8Linear autograd T=33 K=256 N=128")
    rng = np.random.default_rng(24)
    W = _dev((rng.standard_normal((128, 256)) * 0.05).astype(np.float16))
    layer = m8.Int8Linear(W)
    X = _dev(rng.standard_normal((33, 256)).astype(np.float16)).requires_grad_(True)
    Y = layer(X)
    dY = _dev(rng.standard_normal((33, 128)).astype(np.float16))
    Y.backward(dY)
    ref = m8.llmint8_linear_backward_input(dY, layer.Wq, layer.sW)
    assert torch.equal(X.grad.view(torch.int16), ref.view(torch.int16))
    Y2 = m8.llmint8_linear(X.detach(), layer.Wq, layer.sW, 6.0)
    assert torch.equal(Y.detach().view(torch.int16), Y2.view(torch.int16))


# --------------------------------------------------------------------------- bf16 (reading B2 on B1)

def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bf16_host(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _weights_bf16(seed, N, K, sigma=0.02):
    W = workloads.as_bf16_input(workloads.make_weight(workloads.rng_for(seed, 0), N, K, sigma))
    Wq_ref, sW_ref = oracle.quantize_weight(W, "bf16")
    return _dev(Wq_ref), _dev(sW_ref), Wq_ref, sW_ref


@pytest.mark.parametrize("N,K", [(64, 128), (200, 336), (8, 16), (1000, 1040), (11008, 4096)])
def test_dequantize_transposed_bf16_bit_exact(N, K):
    _say(f"dequantize_weight_t_ex bf16 N={N} K={K}")
    Wq, sW, Wq_ref, sW_ref = _weights_bf16(23, N, K)
    WdT = _bf16_host(m8.llmint8_dequantize_weight_t_ex(Wq, sW, dtype=torch.bfloat16))
    ref = oracle.dequantize_weight(Wq_ref, sW_ref, "bf16").T
    assert np.array_equal(WdT, np.ascontiguousarray(ref))


@pytest.mark.parametrize("N,K,dtype", [(520, 272, "f16"), (1000, 1040, "f16"), (72, 16, "f16"),
                                       (2056, 4112, "bf16"), (11008, 4096, "f16")])
def test_on_the_fly_dequantization_bit_exact(N, K, dtype):
    """dY one-hot over a permutation of the weight rows: dX row t = Wdeq row perm[t]."""
    _say(f"backward one-hot N={N} K={K} {dtype}")
    Wq, sW, Wq_ref, sW_ref = _weights(27, N, K)
    rng = np.random.default_rng(N + K)
    T = min(N, 2048)
    perm = rng.permutation(N)[:T]
    one = np.uint16(0x3C00 if dtype == "f16" else 0x3F80)      # 1.0 in fp16 / bf16
    dY = np.zeros((T, N), np.uint16)
    dY[np.arange(T), perm] = one
    dYd = _dev(dY).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    dX = _host(m8.llmint8_linear_backward_input_ex(dYd, Wq, sW).view(torch.int16)).view(np.uint16)
    ref = oracle.dequantize_weight(Wq_ref, sW_ref, dtype)
    ref = ref.view(np.uint16) if ref.dtype != np.uint16 else ref
    assert np.array_equal(dX, ref[perm]), "on-the-fly dequantized operand differs"


@pytest.mark.parametrize("T,K,N", [(16, 1024, 1024), (37, 336, 200), (300, 512, 264),
                                   (1, 4096, 4096), (257, 144, 520), (5, 16, 8)])
def test_backward_input_bf16_parity(T, K, N):
    from parity_util import check_y
    _say(f"backward_input_ex bf16 T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = _weights_bf16(24, N, K)
    dY = workloads.as_bf16_input(workloads.make_output_grad(24, T, N))
    dX = _bf16_host(m8.llmint8_linear_backward_input_ex(_bf16_dev(dY), Wq, sW))
    ref = oracle.linear_backward_input(dY, Wq_ref, sW_ref, "bf16")
    check_y(dX, ref, "bf16")
    # the fp16 entry through _ex equals the plain entry point
    dYh = workloads.make_output_grad(24, T, N)
    Wq2, sW2, _, _ = _weights(24, N, K)
    a = _host(m8.llmint8_linear_backward_input_ex(_dev(dYh), Wq2, sW2)).view(np.uint16)
    b = _host(m8.llmint8_linear_backward_input(_dev(dYh), Wq2, sW2)).view(np.uint16)
    assert np.array_equal(a, b)


def test_backward_input_bf16_prefill_layer_sampled_rows():
    from parity_util import check_y
    w = workloads.CONFIGS["prefill"]
    _say(f"backward_input_ex bf16 prefill layer T={w.T} K={w.K} N={w.N}")
    Wq, sW, Wq_ref, sW_ref = _weights_bf16(w.seed, w.N, w.K, w.sigma)
    dY = workloads.as_bf16_input(workloads.make_output_grad(w.seed, w.T, w.N))
    dX = _bf16_host(m8.llmint8_linear_backward_input_ex(_bf16_dev(dY), Wq, sW))
    rows = np.unique(np.concatenate([np.sort(np.random.default_rng(9).choice(w.T, 32, replace=False)),
                                     [0, w.T - 1]]))
    ref = oracle.linear_backward_input(dY[rows], Wq_ref, sW_ref, "bf16")
    check_y(np.ascontiguousarray(dX[rows]), ref, "bf16")


def test_int8linear_bf16_autograd_uses_the_kernels():
    _say("Int8Linear bf16 autograd")
    N, K, T = 264, 512, 24
    W = workloads.as_bf16_input(workloads.make_weight(workloads.rng_for(25, 0), N, K, 0.05))
    layer = m8.Int8Linear(_bf16_dev(W), threshold=6.0)
    X = workloads.as_bf16_input(workloads.make(
        workloads.Workload("g", T=T, K=K, N=N, sigma=0.05, n_out=3, lo=20, hi=60, threshold=6.0,
                           seed=25), with_weight=False)[1])
    Xd = _bf16_dev(X).requires_grad_(True)
    Y = layer(Xd.reshape(2, T // 2, K))
    gY = _bf16_dev(workloads.as_bf16_input(workloads.make_output_grad(25, T, N))).reshape(2, T // 2, N)
    Y.backward(gY)
    got = _bf16_host(Xd.grad.detach().contiguous())
    want = _bf16_host(m8.llmint8_linear_backward_input_ex(gY.reshape(T, N).contiguous(),
                                                          layer.Wq, layer.sW))
    assert np.array_equal(got, want)


def test_backward_input_maximum_n():
    """N = 65536, the largest reduction length the input gradient takes."""
    from parity_util import check_y
    T, K, N = 9, 64, 65536
    _say(f"backward_input T={T} K={K} N={N}")
    Wq, sW, Wq_ref, sW_ref = _weights(26, N, K)
    dY = workloads.make_output_grad(26, T, N)
    dX = _host(m8.llmint8_linear_backward_input(_dev(dY), Wq, sW))
    check_y(dX, oracle.linear_backward_input(dY, Wq_ref, sW_ref), "f16")


@pytest.mark.parametrize("i", range(40))
def test_backward_input_random_sweep(i):
    """Seeded random shapes (T up to 600, K up to 4800, N up to 2400 in steps
    of 8) in fp16 and bf16: the transposed dequantized weight bit-exact and dX
    within the bar of its type."""
    from parity_util import check_y
    rng = np.random.default_rng(8000 + i)
    T = int(rng.integers(1, 601))
    K = 16 * int(rng.integers(1, 301))
    N = 8 * int(rng.integers(1, 301))
    bf16 = bool(rng.random() < 0.5)
    _say(f"backward sweep {i}: T={T} K={K} N={N} bf16={bf16}")
    if bf16:
        Wq, sW, Wq_ref, sW_ref = _weights_bf16(8100 + i, N, K)
        dY = workloads.as_bf16_input(workloads.make_output_grad(8100 + i, T, N))
        WdT = _bf16_host(m8.llmint8_dequantize_weight_t_ex(Wq, sW, dtype=torch.bfloat16))
        assert np.array_equal(WdT, np.ascontiguousarray(oracle.dequantize_weight(Wq_ref, sW_ref, "bf16").T))
        dX = _bf16_host(m8.llmint8_linear_backward_input_ex(_bf16_dev(dY), Wq, sW))
        check_y(dX, oracle.linear_backward_input(dY, Wq_ref, sW_ref, "bf16"), "bf16")
    else:
        Wq, sW, Wq_ref, sW_ref = _weights(8100 + i, N, K)
        dY = workloads.make_output_grad(8100 + i, T, N)
        WdT = _host(m8.llmint8_dequantize_weight_t(Wq, sW)).view(np.uint16)
        assert np.array_equal(WdT, np.ascontiguousarray(oracle.dequantize_weight(Wq_ref, sW_ref).T).view(np.uint16))
        dX = _host(m8.llmint8_linear_backward_input(_dev(dY), Wq, sW))
        assert oracle.parity_error(dX, oracle.linear_backward_input(dY, Wq_ref, sW_ref)) <= DX_TOL
