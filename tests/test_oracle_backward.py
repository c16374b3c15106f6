"""Pins for the oracle's input gradient through the frozen int8 layer.

Sources (page title, section): "Hugging Face Quantization with bitsandbytes:
4-bit & 8-bit Models Explained", the quick comparison table (an int8 model is
frozen and an adapter is trained on top) and section 6 (gradients flow through
the frozen quantized weights); "bitsandbytes" (mining glossary), "Where it
fits in the stack" (weights are dequantized per operation).

What is pinned, and by what other than the oracle itself:
* P12  every entry of Wdeq and dX equals an independent pure-Python evaluation
       (exact rationals, struct rounding) on tiny shapes;
* P13  integer weights whose rows reach +-127 dequantize to themselves, and
       integer gradients then give the exact integer product;
* P14  the adjoint identity <dY, X . Wdeq^T> = <dX, X> (catches a transposed
       or mis-indexed operand), within the bound fp16 rounding of dX allows;
* P15  the forward's outlier operand is the same dequantized weight, column by
       column, and a zero-scale row contributes nothing;
* the planted mistakes listed in the last test each fail one of these.
"""
from __future__ import annotations

import numpy as np
import pytest

import brute_llmint8 as brute
import oracle

SPECIAL = [0.0, 0.5, -0.5, 1.0, -1.0, 2.5, -3.5, 6.0, -127.0, 0.0999755859375]


def _draw(rng, shape, scale=1.0):
    x = rng.standard_normal(shape) * scale
    flat = x.reshape(-1)
    pick = rng.random(flat.shape) < 0.2
    flat[pick] = rng.choice(SPECIAL, size=int(pick.sum()))
    return x.astype(np.float16)


def _tiny_cases():
    rng = np.random.default_rng(12)
    cases = []
    for T in (1, 2, 4):
        for N in (1, 3, 4):
            for K in (1, 5, 8):
                W = _draw(rng, (N, K), 0.5)
                dY = _draw(rng, (T, N), 2.0)
                cases.append((dY, W))
    return cases


def _check_twin(fn=None):
    bw = fn or oracle.linear_backward_input
    bad = []
    for dY, W in _tiny_cases():
        Wq, sW = oracle.quantize_weight(W)
        Wd_ref, dX_ref = brute.backward_input(dY.astype(float).tolist(), Wq.astype(int).tolist(),
                                              sW.astype(float).tolist())
        if oracle.dequantize_weight(Wq, sW).astype(float).tolist() != Wd_ref:
            bad.append(("Wdeq", W.shape))
        dX = bw(dY, Wq, sW).astype(float).tolist()
        if dX != dX_ref:
            bad.append(("dX", dY.shape, W.shape))
    return bad


def test_p12_bruteforce_twin_tiny_shapes():
    """P12: Wdeq and dX equal an independent exact evaluation (T<=4, N<=4, K<=8)."""
    bad = _check_twin()
    assert not bad, bad[:3]


def _bf16(a):
    b = np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)             # truncation: exact bf16 inputs


def _check_twin_bf16(bw=None, deq=None):
    bw = bw or oracle.linear_backward_input
    deq = deq or oracle.dequantize_weight
    bad = []
    for dY, W in _tiny_cases():
        Wb, dYb = _bf16(W.astype(np.float32)), _bf16(dY.astype(np.float32))
        Wq, sW = oracle.quantize_weight(Wb, "bf16")
        dY_vals = oracle.bf16_bits_to_f32(dYb).astype(float).tolist()
        Wd_ref, dX_ref = brute.backward_input(dY_vals, Wq.astype(int).tolist(),
                                              sW.astype(float).tolist(), to_bf16=True)
        if oracle.bf16_bits_to_f32(deq(Wq, sW, "bf16")).astype(float).tolist() != Wd_ref:
            bad.append(("Wdeq", W.shape))
        if oracle.bf16_bits_to_f32(bw(dYb, Wq, sW, "bf16")).astype(float).tolist() != dX_ref:
            bad.append(("dX", dY.shape, W.shape))
    return bad


def test_p12_bf16_twin_tiny_shapes():
    """P12 with bf16 activations (B2): Wdeq and dX rounded to bf16 equal the exact twin."""
    bad = _check_twin_bf16()
    assert not bad, bad[:3]


def test_p12_bf16_planted_mistakes_are_caught():
    """Rounding Wdeq through fp16, or the sum to fp16, in bf16 mode fails the bf16 twin."""
    good_deq = oracle.dequantize_weight

    def deq_via_fp16(Wq, sW, dtype="f16"):
        d = good_deq(Wq, sW, "f16").astype(np.float32)
        return oracle.f32_to_bf16_bits(d) if dtype == "bf16" else d.astype(np.float16)

    def bw_fp16_sum(dY, Wq, sW, dtype="f16"):
        Wd = oracle.bf16_bits_to_f32(good_deq(Wq, sW, "bf16")).astype(np.float64)
        out = (oracle.bf16_bits_to_f32(dY).astype(np.float64) @ Wd).astype(np.float16)
        return oracle.f32_to_bf16_bits(out.astype(np.float32))

    def bw_via(deq):
        def f(dY, Wq, sW, dtype="f16"):
            Wd = oracle.bf16_bits_to_f32(deq(Wq, sW, "bf16")).astype(np.float64)
            return oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f32(dY).astype(np.float64) @ Wd)
        return f

    assert _check_twin_bf16(bw=bw_via(deq_via_fp16), deq=deq_via_fp16)
    assert _check_twin_bf16(bw=bw_fp16_sum)


def _p13(fn=None):
    bw = fn or oracle.linear_backward_input
    rng = np.random.default_rng(13)
    T, N, K = 6, 9, 11
    W = rng.integers(-127, 128, size=(N, K))
    W[np.arange(N), rng.integers(0, K, N)] = 127 * rng.choice([-1, 1], N)
    Wq, sW = oracle.quantize_weight(W.astype(np.float16))
    assert np.array_equal(Wq, W) and np.all(sW == 127)
    assert np.array_equal(oracle.dequantize_weight(Wq, sW).astype(np.int64), W)
    dY = rng.integers(-2, 3, size=(T, N))
    exact = dY @ W                                   # |exact| <= 9*2*127 < 2048: exact in fp16
    return np.array_equal(bw(dY.astype(np.float16), Wq, sW).astype(np.int64), exact)


def test_p13_integer_weights_dequantize_exactly():
    """P13: integer weights reaching +-127 per row are their own dequantization; dX is the integer product."""
    assert _p13()


def _p14(fn=None, shapes=((7, 12, 10), (3, 33, 5), (8, 8, 8))):
    bw = fn or oracle.linear_backward_input
    rng = np.random.default_rng(14)
    for T, N, K in shapes:
        W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
        Wq, sW = oracle.quantize_weight(W)
        Wd = oracle.dequantize_weight(Wq, sW).astype(np.float64)
        X = rng.standard_normal((T, K))
        dY = rng.standard_normal((T, N)).astype(np.float16).astype(np.float64)
        dX = bw(dY.astype(np.float16), Wq, sW).astype(np.float64)
        lhs = float(np.sum(dY * (X @ Wd.T)))         # <dY, X Wdeq^T>, with the forward's orientation
        rhs = float(np.sum(dX * X))                  # <dX, X>
        bound = float(np.sum(np.abs(dX * X))) * 2.0 ** -10 + 1e-9
        if not abs(lhs - rhs) <= bound:
            return False
    return True


def test_p14_adjoint_identity():
    """P14: <dY, X Wdeq^T> = <dX, X> up to the fp16 rounding of dX."""
    assert _p14()


def test_p14_adjoint_of_exact_forward():
    """P14 on the forward itself: with inputs the int8 path reproduces exactly, the
    forward's Y and the backward's dX are adjoint maps of the same weight."""
    rng = np.random.default_rng(141)
    T, N, K = 5, 7, 9
    X = rng.integers(-127, 128, size=(T, K))
    X[:, 0] = 127
    W = rng.integers(-127, 128, size=(N, K))
    W[:, 1] = -127
    Wq, sW = oracle.quantize_weight(W.astype(np.float16))
    st = oracle.linear(X.astype(np.float16), Wq, sW, np.inf)
    dY = rng.integers(-3, 4, size=(T, N))
    dX = oracle.linear_backward_input(dY.astype(np.float16), Wq, sW).astype(np.int64)
    Y = st.C.astype(np.int64)                        # = X W^T exactly (scales are 127)
    assert np.array_equal(Y, X @ W.T)
    assert int(np.sum(dY * Y)) == int(np.sum(dX * X))


def _p15(deq=None):
    deq = deq or oracle.dequantize_weight
    rng = np.random.default_rng(15)
    T, N, K = 4, 6, 40
    X = rng.standard_normal((T, K)).astype(np.float16)
    X[1, [3, 17, 29]] = [30.0, -22.0, 41.0]
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[2] = 0.0                                       # a zero row: scale 0, codes 0
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, 6.0)
    Wdeq = deq(Wq, sW)
    return (np.array_equal(st.Wd.view(np.uint16), Wdeq[:, st.idx].view(np.uint16))
            and not np.any(Wdeq[2].astype(np.float32)))


def test_p15_same_dequantization_as_forward_outliers():
    """P15: the forward's outlier operand is the dequantized weight at the outlier columns;
    a zero-scale row dequantizes to zeros."""
    assert _p15()


def test_zero_and_empty_shapes():
    Wq = np.zeros((3, 16), np.int8)
    sW = np.zeros(3, np.float32)
    assert oracle.linear_backward_input(np.zeros((0, 3), np.float16), Wq, sW).shape == (0, 16)
    dX = oracle.linear_backward_input(np.ones((2, 3), np.float16), Wq, sW)
    assert dX.shape == (2, 16) and not np.any(dX.astype(np.float32))


def test_planted_mistakes_are_caught():
    """Each plausible mistake in the backward fails at least one pin above."""
    good = oracle.linear_backward_input
    deq = oracle.dequantize_weight

    def transposed(dY, Wq, sW):                      # uses W^T where W is meant (square only)
        Wd = deq(Wq, sW).astype(np.float64)
        return (dY.astype(np.float64) @ Wd.T).astype(np.float16)

    def no_div(dY, Wq, sW):
        Wd = (Wq.astype(np.float32) * sW[:, None]).astype(np.float16).astype(np.float64)
        with np.errstate(over="ignore"):
            return (dY.astype(np.float64) @ Wd).astype(np.float16)

    def no_scale(dY, Wq, sW):
        Wd = (Wq.astype(np.float32) / np.float32(127)).astype(np.float16).astype(np.float64)
        with np.errstate(over="ignore"):
            return (dY.astype(np.float64) @ Wd).astype(np.float16)

    def fp16_sum(dY, Wq, sW):                        # accumulates in fp16
        Wd = deq(Wq, sW)
        out = np.zeros((dY.shape[0], Wd.shape[1]), np.float16)
        for n in range(Wd.shape[0]):
            out = (out + dY[:, n:n + 1] * Wd[n:n + 1, :]).astype(np.float16)
        return out

    def negated(dY, Wq, sW):
        return (-good(dY, Wq, sW).astype(np.float32)).astype(np.float16)

    def square_p14(fn):
        return _p14(fn, shapes=((8, 8, 8), (5, 6, 6)))

    def caught(fn):
        checks = [lambda: not _check_twin(fn), lambda: _p13(fn), lambda: square_p14(fn)]
        for c in checks:
            try:
                if not c():
                    return True
            except (AssertionError, ValueError):
                return True
        return False

    assert not caught(good)
    mutants = {"transposed": transposed, "no /127": no_div, "no row scale": no_scale,
               "fp16 accumulation": fp16_sum, "sign": negated}
    result = {k: caught(f) for k, f in mutants.items()}
    assert all(result.values()), result

    def deq_no_div(Wq, sW):
        return (Wq.astype(np.float32) * sW[:, None]).astype(np.float16)
    assert not _p15(deq_no_div)


def test_kernel_dequant_multiply_form_is_exact():
    """The kernels dequantize with one fp32 multiply by fl32(1/127); for every scale
    llmint8_quantize_weight can produce (a positive fp16 value) and every code, the fp16
    result equals the one of the fp32 division that the method defines."""
    codes = np.arange(1, 0x7C00, dtype=np.uint16)
    b = codes.view(np.float16).astype(np.float32)
    q = np.arange(-127, 128, dtype=np.float32)
    p = (q[None, :] * b[:, None]).astype(np.float32)
    div = (p / np.float32(127.0)).astype(np.float16)
    mul = (p * np.float32(1.0 / 127.0)).astype(np.float32).astype(np.float16)
    assert np.array_equal(div.view(np.uint16), mul.view(np.uint16))


def _f32_to_bf16_bits_rne(x32):
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_kernel_dequant_multiply_form_is_exact_bf16():
    """bf16 compute type: for every positive finite bf16 scale and every code, rounding
    fl32(fl32(q * b) * fl32(1/127)) to bf16 gives the bf16 rounding of the division."""
    codes = np.arange(1, 0x7F80, dtype=np.uint32)
    b = (codes << 16).view(np.float32)
    q = np.arange(-127, 128, dtype=np.float32)
    p = (q[None, :] * b[:, None]).astype(np.float32)      # exact: 8-bit times 8-bit significands
    div = _f32_to_bf16_bits_rne((p / np.float32(127.0)).astype(np.float32))
    mul = _f32_to_bf16_bits_rne((p * np.float32(1.0 / 127.0)).astype(np.float32))
    assert np.array_equal(div, mul)


def test_kernel_dequant_multiply_form_single_rounding_fp16():
    """fp16 with the second product rounded to fp16 once (no fp32 rounding between, as a
    fused mixed-precision multiply-add gives): still the fp16 rounding of the division,
    for every positive fp16 scale and every code."""
    codes = np.arange(1, 0x7C00, dtype=np.uint16)
    b = codes.view(np.float16).astype(np.float32)
    q = np.arange(-127, 128, dtype=np.float32)
    p = (q[None, :] * b[:, None]).astype(np.float32)      # exact in fp32
    div = (p / np.float32(127.0)).astype(np.float16)
    # p (<= 19 significant bits) times fl32(1/127) (24 bits) is exact in binary64
    once = (p.astype(np.float64) * np.float64(np.float32(1.0 / 127.0))).astype(np.float16)
    assert np.array_equal(div.view(np.uint16), once.view(np.uint16))
