"""Pins for the oracle's bf16 activation mode and the fused bias.

Sources (page title, section): "Hugging Face Quantization with bitsandbytes:
4-bit & 8-bit Models Explained", section 5 (storage type and compute type are
separate choices, bfloat16 preferred where the hardware has it);
"bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit Depths"
(Linear8bitLt replaces a linear layer, which has a bias).

* P21  the oracle's bf16 roundings (from fp32 and from float64) equal torch's
       fp32 -> bfloat16 conversion and an exact-rational rounding;
* P22  every stage of the bf16 forward, with and without bias, equals the
       independent pure-Python twin on tiny shapes;
* P23  on inputs exact in both fp16 and bf16 the quantization stages (outlier
       set, codes, row and column maxima, C) do not depend on the type;
* P24  with integer inputs that quantize exactly, Y is C + bias exactly;
* planted mistakes each fail one of these.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import brute_llmint8 as brute
import oracle

torch = pytest.importorskip("torch")


def _bf16(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _vals(bits):
    return oracle.bf16_bits_to_f32(bits).astype(float)


def test_p21_bf16_rounding_matches_torch_and_exact_rounding():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38, 1e-39, -7e-42]])
    x32 = x.astype(np.float32)
    ours = oracle.f32_to_bf16_bits(x32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # float64 -> bf16 in one rounding, against exact rationals
    y = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    y = np.concatenate([y, [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 2.0 ** -130]])
    got = _vals(oracle.f64_to_bf16_bits(y))
    want = [brute.bf16_of_fraction(Fraction(float(v))) for v in y]
    assert got.tolist() == want


def _tiny_bf16_cases():
    rng = np.random.default_rng(22)
    special = [0.0, 0.5, -2.5, 3.5, 6.0, -6.0, 127.0, 5.96875, 100.0]
    cases = []
    for T in (1, 2, 3):
        for K in (1, 4, 7):
            for N in (1, 3):
                X = rng.standard_normal((T, K)) * 3
                X[rng.random((T, K)) < 0.25] = rng.choice(special)
                W = rng.standard_normal((N, K)) * 0.3
                bias = rng.standard_normal(N) if (T + K + N) % 2 else None
                cases.append((_bf16(X), _bf16(W), None if bias is None else _bf16(bias),
                              [6.0, 0.75, math.inf][(T * K * N) % 3]))
    return cases


def _twin_bad(ora_linear=None):
    lin = ora_linear or oracle.linear
    bad = []
    for X, W, bias, thr in _tiny_bf16_cases():
        Wq, sW = oracle.quantize_weight(W, dtype="bf16")
        st = lin(X, Wq, sW, thr, dtype="bf16", bias=bias)
        ref = brute.forward(_vals(X).tolist(), _vals(W).tolist(), thr, bf16_io=True,
                            bias=None if bias is None else _vals(bias).tolist())
        if (list(st.idx) != ref["outliers"] or Wq.tolist() != ref["Wq"] or st.Xq.tolist() != ref["Xq"]
                or st.C.tolist() != ref["C"]):
            bad.append(("stages", X.shape, W.shape))
        elif _vals(st.Wd).tolist() != ref["Wd"] or _vals(st.Y).tolist() != ref["Y"]:
            bad.append(("Wd/Y", X.shape, W.shape, bias is not None))
    return bad


def test_p22_bf16_and_bias_equal_the_twin():
    bad = _twin_bad()
    assert not bad, bad[:3]


def test_p22_fp16_bias_equals_the_twin():
    rng = np.random.default_rng(221)
    for _ in range(12):
        X = (rng.standard_normal((3, 6)) * 4).astype(np.float16)
        W = (rng.standard_normal((4, 6)) * 0.2).astype(np.float16)
        bias = rng.standard_normal(4).astype(np.float16)
        Wq, sW = oracle.quantize_weight(W)
        st = oracle.linear(X, Wq, sW, 6.0, bias=bias)
        ref = brute.forward(X.astype(float).tolist(), W.astype(float).tolist(), 6.0,
                            bias=bias.astype(float).tolist())
        assert st.Y.astype(float).tolist() == ref["Y"]


def test_p23_quantization_stages_do_not_depend_on_the_type():
    rng = np.random.default_rng(23)
    # values with at most 8 significant bits and within fp16 range: exact in both types
    X = (rng.integers(-255, 256, (9, 40)) * 2.0 ** rng.integers(-6, 2, (9, 40))).astype(np.float32)
    X[:, 7] = 48.0
    W = (rng.integers(-255, 256, (11, 40)) * 2.0 ** -8).astype(np.float32)
    X16, Xb = X.astype(np.float16), _bf16(X)
    W16, Wb = W.astype(np.float16), _bf16(W)
    assert np.array_equal(X16.astype(np.float32), X) and np.array_equal(_vals(Xb), X)
    a = oracle.linear(X16, *oracle.quantize_weight(W16), 6.0)
    b = oracle.linear(Xb, *oracle.quantize_weight(Wb, dtype="bf16"), 6.0, dtype="bf16")
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.Xq, b.Xq)
    assert np.array_equal(a.aX, b.aX) and np.array_equal(a.C, b.C)
    assert np.array_equal(oracle.quantize_weight(W16)[0], oracle.quantize_weight(Wb, dtype="bf16")[0])


def _p24(ora_linear=None):
    lin = ora_linear or oracle.linear
    rng = np.random.default_rng(24)
    T, K, N = 4, 16, 6
    X = rng.integers(-127, 128, (T, K)).astype(np.float32)
    X[:, 0] = 127
    W = rng.integers(-127, 128, (N, K)).astype(np.float32)
    W[:, 1] = -127
    bias = rng.integers(-100, 100, N).astype(np.float32)
    ok = True
    for dtype, conv in (("f16", lambda v: v.astype(np.float16)), ("bf16", _bf16)):
        Wq, sW = oracle.quantize_weight(conv(W), dtype=dtype)
        st = lin(conv(X), Wq, sW, math.inf, dtype=dtype, bias=conv(bias))
        exact = (X.astype(np.int64) @ W.T.astype(np.int64)) + bias.astype(np.int64)[None, :]
        Y = st.Y.astype(np.float64) if dtype == "f16" else _vals(st.Y)
        want = exact.astype(np.float64)
        if dtype == "bf16":
            want = _vals(oracle.f64_to_bf16_bits(want))
        else:
            want = want.astype(np.float16).astype(np.float64)
        ok = ok and np.array_equal(Y, want)
    return ok


def test_p24_integer_inputs_give_c_plus_bias():
    assert _p24()


def test_planted_mistakes_are_caught(monkeypatch):
    mod = oracle.llmint8_oracle
    good_output = mod.output

    def bias_after_rounding(C, aX, sW, Xo, Wd, dtype="f16", bias=None):
        Y = good_output(C, aX, sW, Xo, Wd, dtype, None)
        if bias is None:
            return Y
        if dtype == "bf16":
            return oracle.f64_to_bf16_bits(_vals(Y) + _vals(bias)[None, :])
        return (Y.astype(np.float64) + bias.astype(np.float64)[None, :]).astype(np.float16)

    def bias_dropped(C, aX, sW, Xo, Wd, dtype="f16", bias=None):
        return good_output(C, aX, sW, Xo, Wd, dtype, None)

    def bf16_truncated(x32):
        return (np.asarray(x32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)

    caught = {}
    for label, (name, fn) in {"bias after rounding": ("output", bias_after_rounding),
                              "bias dropped": ("output", bias_dropped),
                              "bf16 truncation": ("f32_to_bf16_bits", bf16_truncated)}.items():
        with monkeypatch.context() as m:
            m.setattr(mod, name, fn)
            try:
                caught[label] = bool(_twin_bad()) or not _p24()
            except (AssertionError, ValueError):
                caught[label] = True
    assert all(caught.values()), caught
