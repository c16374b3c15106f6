"""Pins for the oracle's 4-bit weight path (NF4 / FP4 code books, blockwise
codes, dequantization, the decode-shaped linear).

Sources (page title, section): "bitsandbytes" (glossary), "What it provides"
(FP4 and NF4, blockwise scaling, 16-bit compute with weights dequantized on
the fly); "Hugging Face
Quantization with bitsandbytes ...", section 4 (NF4 fitted to normally
distributed weights, FP4 a generic 4-bit float).

* P25  the NF4 book equals one built from normal quantiles found by bisection
       on math.erfc (no library inverse), and its levels sit at evenly spaced
       probabilities on each side of zero;
* P26  the FP4 book equals E2M1 decoded through fp32 bit patterns, and its
       magnitudes are the E2M1 value set scaled to a largest value of 1;
* P27  blockwise codes, maxima and dequantized values equal the pure-Python twin
       (fp16 and bf16 inputs, ragged last blocks, zero blocks, exact midpoints);
* P28  every code is the nearest level (up to one fp32 step at a midpoint);
* P29  the reconstruction error is at most half the widest gap between levels
       times the block maximum, plus the 16-bit rounding;
* P30  the linear equals the twin's exact sum with one rounding; weights whose
       magnitudes all equal their block maximum dequantize to +-a exactly, so
       integer activations give a closed-form product;
* planted mistakes each fail one of these.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import brute_llmint8 as brute
import oracle
import workloads

BOOKS = {"nf4": brute.nf4_book, "fp4": brute.fp4_book}


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_p25_nf4_book_matches_bisection_quantiles():
    assert np.array_equal(_bits(oracle.code_book("nf4")), _bits(brute.nf4_book()))


def test_p25_nf4_book_shape_and_probabilities():
    b = oracle.code_book("nf4").astype(float)
    assert np.all(np.diff(b) > 0)
    assert b[0] == -1.0 and b[7] == 0.0 and b[15] == 1.0
    assert np.sum(b < 0) == 7 and np.sum(b > 0) == 8
    d = brute.normal_quantile(oracle.NF4_P_MAX)
    pos = sorted(brute.phi(v * d) for v in b[b > 0])
    neg = sorted(brute.phi(-v * d) for v in b[b < 0])
    for side, count in ((pos, 8), (neg, 7)):
        step = (oracle.NF4_P_MAX - 0.5) / count
        want = [0.5 + step * (i + 1) for i in range(count)]
        assert np.allclose(side, want, atol=1e-6)


def test_p26_fp4_book_is_e2m1():
    book = oracle.code_book("fp4")
    assert np.array_equal(_bits(book), _bits(brute.fp4_book()))
    mags = sorted(set(np.abs(book.astype(float)) * 6.0))
    assert np.allclose(mags, [0, 0.5, 1, 1.5, 2, 3, 4, 6], atol=1e-6)
    assert all(math.copysign(1.0, book[c]) < 0 for c in range(8, 16))
    assert all(math.copysign(1.0, book[c]) > 0 for c in range(8))


def _vals16(a, dtype):
    return oracle.bf16_bits_to_f32(a).astype(float) if dtype == "bf16" else a.astype(float)


def _tiny_inputs():
    rng = np.random.default_rng(27)
    cases = []
    for n, block in ((2, 64), (64, 64), (100, 64), (130, 64), (256, 128), (258, 128), (512, 256)):
        w = (rng.standard_normal(n) * 0.05).astype(np.float16)
        if n >= 128:
            w[64:128] = 0                      # a zero block (for block 64) / half block
        cases.append((w, block))
    # exact midpoints: a block whose maximum is 1 and whose entries sit on midpoints
    for q in ("nf4", "fp4"):
        _, mids = oracle.quantize_levels(q)
        w = np.zeros(64, np.float32)
        w[0] = 1.0
        m16 = mids.astype(np.float16)
        keep = m16.astype(np.float32) == mids       # midpoints exact in fp16
        w[1:1 + int(keep.sum())] = mids[keep]
        cases.append((w.astype(np.float16), 64))
    return cases


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_p27_codes_and_dequantization_match_twin(quant_type, dtype):
    book = BOOKS[quant_type]()
    for w16, block in _tiny_inputs():
        w = workloads.as_bf16_input(w16) if dtype == "bf16" else w16
        vals = list(_vals16(w, dtype))
        packed, a = oracle.quantize_4bit(w, block, quant_type, dtype)
        p_ref, a_ref = brute.quantize_4bit(vals, block, book)
        assert packed.tolist() == p_ref
        assert a.tolist() == a_ref
        d = oracle.dequantize_4bit(packed, a, block, quant_type, len(vals), dtype)
        d_ref = brute.dequantize_4bit(p_ref, a_ref, block, book, len(vals), dtype == "bf16")
        assert list(_vals16(d, dtype)) == d_ref


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_p28_codes_are_nearest_levels(quant_type):
    rng = np.random.default_rng(28)
    book = oracle.code_book(quant_type).astype(float)
    w = rng.uniform(-1, 1, 8192).astype(np.float16)
    w[::64] = 1.0                                  # every block's maximum is 1: x_n = w exactly
    packed, a = oracle.quantize_4bit(w, 64, quant_type)
    assert np.all(a == 1.0)
    got = book[oracle.unpack_4bit(packed, w.size)]
    dist = np.abs(w.astype(float)[:, None] - np.unique(book)[None, :]).min(axis=1)
    assert np.all(np.abs(w.astype(float) - got) <= dist + 2.0 ** -24)
    if quant_type == "fp4":
        assert not np.any(oracle.unpack_4bit(packed, w.size) == 8)   # zero is the +0 code


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_p29_reconstruction_error_bound(quant_type):
    rng = np.random.default_rng(29)
    book = np.unique(oracle.code_book(quant_type).astype(float))
    half_gap = np.max(np.diff(book)) / 2
    w = (rng.standard_normal(64 * 200) * 0.02).astype(np.float16)
    packed, a = oracle.quantize_4bit(w, 64, quant_type)
    d = oracle.dequantize_4bit(packed, a, 64, quant_type, w.size).astype(float)
    a_el = np.repeat(a.astype(float), 64)
    assert np.all(np.abs(d - w.astype(float)) <= a_el * half_gap * (1 + 1e-6) + 2.0 ** -11 * a_el)


def _linear_cases():
    rng = np.random.default_rng(30)
    for T, K, N, block in ((1, 64, 3, 64), (2, 128, 2, 64), (3, 64, 4, 32), (1, 256, 1, 128)):
        X = rng.standard_normal((T, K)).astype(np.float16)
        W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
        b = (rng.standard_normal(N) * 0.5).astype(np.float16)
        yield X, W, b, block


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_p30_linear_matches_twin(quant_type, dtype):
    book = BOOKS[quant_type]()
    for X, W, b, block in _linear_cases():
        if dtype == "bf16":
            X, W, b = (workloads.as_bf16_input(v) for v in (X, W, b))
        N, K = W.shape
        packed, a = oracle.quantize_4bit(W, block, quant_type, dtype)
        for bias in (None, b):
            Y = oracle.linear_4bit(X, packed, a, block, quant_type, N, dtype, bias)
            ref = brute.linear_4bit([list(_vals16(r, dtype)) for r in X], packed.tolist(),
                                    a.tolist(), block, book, N, dtype == "bf16",
                                    None if bias is None else list(_vals16(bias, dtype)))
            assert _vals16(Y, dtype).tolist() == ref


@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_p30_full_magnitude_weights_give_closed_form(quant_type):
    rng = np.random.default_rng(31)
    T, K, N, block = 3, 128, 5, 64
    sign = rng.choice([-1.0, 1.0], size=(N, K))
    scale = 2.0 ** rng.integers(-6, 0, size=(N, K // block))
    W = (sign * np.repeat(scale, block, axis=1)).astype(np.float16)
    X = rng.integers(-8, 9, size=(T, K)).astype(np.float16)
    packed, a = oracle.quantize_4bit(W, block, quant_type)
    Wd = oracle.dequantize_4bit(packed, a, block, quant_type, N * K).reshape(N, K)
    assert np.array_equal(Wd, W)
    Y = oracle.linear_4bit(X, packed, a, block, quant_type, N)
    exact = X.astype(np.float64) @ W.astype(np.float64).T     # integers times powers of two: exact
    assert np.array_equal(Y, exact.astype(np.float16))


def _pins_pass():
    """True when the pins above all hold (used with planted mistakes)."""
    try:
        test_p25_nf4_book_matches_bisection_quantiles()
        test_p25_nf4_book_shape_and_probabilities()
        test_p26_fp4_book_is_e2m1()
        for q in ("nf4", "fp4"):
            for dt in ("f16", "bf16"):
                test_p27_codes_and_dequantization_match_twin(q, dt)
                test_p30_linear_matches_twin(q, dt)
            test_p28_codes_are_nearest_levels(q)
            test_p29_reconstruction_error_bound(q)
            test_p30_full_magnitude_weights_give_closed_form(q)
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    mod = oracle.fourbit_oracle
    good_unpack, good_book, good_levels = mod.unpack_4bit, mod.code_book, mod.quantize_levels

    def swapped_nibbles(packed, n):
        p = np.asarray(packed, dtype=np.uint8).reshape(-1)
        return good_unpack(((p << np.uint8(4)) | (p >> np.uint8(4))).astype(np.uint8), n)

    def ties_up(quant_type):
        order, mids = good_levels(quant_type)
        return order, np.nextafter(mids, np.float32(-np.inf)).astype(np.float32)

    def symmetric_nf4(quant_type):
        if quant_type != "nf4":
            return good_book(quant_type)
        from scipy.stats import norm
        p = (np.arange(16) + 0.5) / 16
        v = norm.ppf(p)
        return (v / v.max()).astype(np.float32)

    def scale_dropped(packed, absmax, block, quant_type, n, dtype="f16"):
        return good_dequant(packed, np.ones_like(np.asarray(absmax)), block, quant_type, n, dtype)

    good_dequant = mod.dequantize_4bit
    mistakes = {"swapped nibbles": ("unpack_4bit", swapped_nibbles),
                "ties to the upper level": ("quantize_levels", ties_up),
                "symmetric NF4 without zero": ("code_book", symmetric_nf4),
                "scale dropped": ("dequantize_4bit", scale_dropped)}
    caught = {}
    for label, (name, fn) in mistakes.items():
        with monkeypatch.context() as m:
            m.setattr(mod, name, fn)
            caught[label] = not _pins_pass()
    with monkeypatch.context() as m:
        m.setattr(mod, "NF4_P_MAX", 0.99)
        caught["wrong NF4 range"] = not _pins_pass()
    assert all(caught.values()), caught
