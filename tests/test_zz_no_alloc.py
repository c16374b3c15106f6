"""The allocation-free forward (llmint8_linear_noalloc, on the library's static
scratch) against the forward with a caller workspace (llmint8_linear_ex), through
the C ABI: bit-identical outputs and the oracle's bar, on calls in a row (each
later one smaller), on the GEMM route, the fused decode route and with bf16 and
a bias; shapes that need more scratch than the library holds are rejected
before anything is enqueued; the calls allocate no device memory."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
import mixed_precision_int8_amd as m8  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(T, K, N, n_out, seed):
    w = workloads.Workload("noalloc", T=T, K=K, N=N, sigma=0.05, n_out=n_out, lo=20.0, hi=60.0,
                           threshold=6.0, seed=seed)
    W, X, _, _ = workloads.make(w)
    return W, X


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m8.load_library()
    assert m8.llmint8_noalloc_scratch_bytes() == 64 << 20
    # (T, K, N, injected outlier columns): GEMM route twice, each call smaller, the
    # first with 600 outlier columns (19 chunks, all held in the scratch); then the
    # fused decode route
    cases = [(300, 2048, 520, 600, 1), (77, 1024, 264, 5, 2), (4, 1024, 300, 3, 3)]
    free_after_first = None
    for i, (T, K, N, n_out, seed) in enumerate(cases):
        _say(f"noalloc T={T} K={K} N={N} n_out={n_out}")
        W, X = _inputs(T, K, N, n_out, seed)
        Wq, sW = m8.llmint8_quantize_weight(torch.from_numpy(W).cuda())
        Xd = torch.from_numpy(X).cuda()
        Y_ws = m8.llmint8_linear_ex(Xd, Wq, sW, 6.0)
        Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        if free_after_first is not None:
            free0 = torch.cuda.mem_get_info()[0]
            alloc0 = torch.cuda.memory_allocated()
        m8.llmint8_linear_noalloc(Xd, Wq, sW, 6.0, Y=Y)
        torch.cuda.synchronize()
        if free_after_first is None:
            free_after_first = torch.cuda.mem_get_info()[0]
        else:
            assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
            assert torch.cuda.memory_allocated() == alloc0
        got, want = Y.cpu().numpy(), Y_ws.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"case {i}: differs"
        Wq_ref, sW_ref = oracle.quantize_weight(W)
        st = oracle.linear(X, Wq_ref, sW_ref, 6.0)
        if i == 0:
            assert st.count >= 600
        err = oracle.parity_error(got, st.Y)
        assert err <= 1e-3, (i, err)


def test_noalloc_bf16_bias_and_limits():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T, K, N = 130, 1024, 200
    _say(f"noalloc bf16 + bias T={T} K={K} N={N}")
    W, X = _inputs(T, K, N, 7, 4)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(workloads.as_bf16_input(a)).view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    b = workloads.make_bias(4, N, bf16=True)
    Wq, sW = m8.llmint8_quantize_weight_ex(bf(W))
    Xd = bf(X)
    bd = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    Y_ws = m8.llmint8_linear_ex(Xd, Wq, sW, 6.0, bias=bd)
    Y = m8.llmint8_linear_noalloc(Xd, Wq, sW, 6.0, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y_ws.view(torch.int16))
    # a shape whose int8 activations alone exceed the scratch: rejected on the host
    lib = m8.load_library()
    T2, K2 = 8192, 8192 + 16
    assert T2 * K2 > m8.llmint8_noalloc_scratch_bytes()
    st = lib.llmint8_linear_noalloc(None, 0, T2, K2, Wq.data_ptr(), sW.data_ptr(), 16, 6.0, None,
                                    None, None)
    assert st == -1                                   # X is NULL: validation first
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = lib.llmint8_linear_noalloc(fake.data_ptr(), 0, T2, K2, Wq.data_ptr(), sW.data_ptr(), 16, 6.0,
                                    None, fake.data_ptr(), None)
    assert st == -3                                   # more than the static scratch holds
