"""Pins for the oracle's blockwise 8-bit codec.

Sources (page title, section): "bitsandbytes" (mining glossary), "What it
provides" (weights quantized in blocks, each with its own scaling factor, so
an outlier only affects its own block); "bitsandbytes: GPU-Accelerated
Inference and Training at Lower Bit Depths", the 8-bit optimizers (block-wise
quantization of the optimizer states).

* P16  codes, block maxima and dequantized values equal an independent
       pure-Python evaluation (struct rounding), fp16 and fp32 inputs, ragged
       last blocks, zero blocks;
* P17  integer blocks that reach +-127 quantize to themselves and dequantize
       back exactly;
* P18  the reconstruction error is at most half a code step of the block
       (plus the output rounding);
* P19  one large value only changes its own block (the pages' reason for
       blocks);
* P20  with the block equal to a weight row the codec is the vector-wise
       weight quantization, which is pinned on its own;
* planted mistakes each fail one of these.
"""
from __future__ import annotations

import numpy as np
import pytest

import brute_llmint8 as brute
import oracle

SPECIAL = [0.0, 0.5, -0.5, 2.5, -3.5, 6.0, -127.0, 1e-3, 300.0]


def _draw(rng, n, dtype):
    x = rng.standard_normal(n) * rng.choice([0.01, 1.0, 50.0])
    pick = rng.random(n) < 0.2
    x[pick] = rng.choice(SPECIAL, size=int(pick.sum()))
    return x.astype(dtype)


def _cases():
    rng = np.random.default_rng(16)
    out = []
    for dtype in (np.float16, np.float32):
        for n in (0, 1, 63, 64, 65, 200, 257):
            for block in (64, 128):
                x = _draw(rng, n, dtype)
                if n > 130:
                    x[64:128] = 0                    # a zero block
                out.append((x, block))
    return out


def _twin_mismatches(qfn=None, dqfn=None):
    qfn = qfn or oracle.quantize_blockwise
    dqfn = dqfn or oracle.dequantize_blockwise
    bad = []
    for x, block in _cases():
        q, a = qfn(x, block)
        q_ref, a_ref = brute.quantize_blockwise(x.astype(float).tolist(), block)
        if q.astype(int).tolist() != q_ref or a.astype(float).tolist() != a_ref:
            bad.append(("codes", x.dtype, x.size, block))
            continue
        to16 = x.dtype == np.float16
        d = dqfn(q, a, block, x.dtype)
        d_ref = brute.dequantize_blockwise(q_ref, a_ref, block, to16)
        if d.astype(float).tolist() != d_ref:
            bad.append(("dequant", x.dtype, x.size, block))
    return bad


def test_p16_bruteforce_twin():
    bad = _twin_mismatches()
    assert not bad, bad[:3]


def _p17(qfn=None, dqfn=None):
    qfn = qfn or oracle.quantize_blockwise
    dqfn = dqfn or oracle.dequantize_blockwise
    rng = np.random.default_rng(17)
    x = rng.integers(-127, 128, size=5 * 64 + 16).astype(np.float32)
    x[::64] = 127 * rng.choice([-1, 1], size=x[::64].shape[0])
    q, a = qfn(x, 64)
    d = dqfn(q, a, 64, np.float32)
    return np.array_equal(q.astype(np.float32), x) and np.all(a == 127) and np.array_equal(d, x)


def test_p17_integer_blocks_are_exact():
    assert _p17()


def _p18(qfn=None, dqfn=None):
    qfn = qfn or oracle.quantize_blockwise
    dqfn = dqfn or oracle.dequantize_blockwise
    rng = np.random.default_rng(18)
    for dtype, block in ((np.float16, 64), (np.float32, 256), (np.float16, 4096)):
        x = _draw(rng, 10000, dtype)
        q, a = qfn(x, block)
        d = dqfn(q, a, block, dtype).astype(np.float64)
        step = np.repeat(a.astype(np.float64), block)[:x.size] / 127.0
        out_ulp = np.abs(d) * (2.0 ** -11 if dtype == np.float16 else 2.0 ** -24) + 2.0 ** -24
        if not np.all(np.abs(d - x.astype(np.float64)) <= step * (0.5 + 1e-6) + out_ulp):
            return False
    return True


def test_p18_reconstruction_error_is_half_a_step():
    assert _p18()


def _p19(qfn=None):
    qfn = qfn or oracle.quantize_blockwise
    rng = np.random.default_rng(19)
    x = rng.standard_normal(1024).astype(np.float16)
    q0, a0 = qfn(x, 128)
    y = x.copy()
    y[300] = 60000.0                                 # block 2
    q1, a1 = qfn(y, 128)
    others = np.ones(1024, bool)
    others[256:384] = False
    return (np.array_equal(q0[others], q1[others]) and np.array_equal(np.delete(a0, 2), np.delete(a1, 2))
            and a1[2] == np.float32(60000.0))


def test_p19_an_outlier_only_changes_its_block():
    assert _p19()


def test_p20_row_blocks_are_the_vectorwise_weight_quantization():
    rng = np.random.default_rng(20)
    W = (rng.standard_normal((37, 192)) * 0.05).astype(np.float16)
    W[5] = 0
    Wq, sW = oracle.quantize_weight(W)
    q, a = oracle.quantize_blockwise(W, 192)
    assert np.array_equal(q.reshape(W.shape), Wq) and np.array_equal(a, sW)
    assert np.array_equal(oracle.dequantize_blockwise(q, a, 192).reshape(W.shape).view(np.uint16),
                          oracle.dequantize_weight(Wq, sW).view(np.uint16))


def test_empty_input():
    q, a = oracle.quantize_blockwise(np.zeros(0, np.float16), 64)
    assert q.shape == (0,) and a.shape == (0,)
    assert oracle.dequantize_blockwise(q, a, 64).shape == (0,)


def test_planted_mistakes_are_caught():
    good_q, good_dq = oracle.quantize_blockwise, oracle.dequantize_blockwise

    def global_absmax(x, block):
        flat = np.asarray(x).reshape(-1)
        q, a = good_q(flat, max(flat.size, 1))
        nb = -(-flat.size // block)
        return q, np.full(nb, a[0] if a.size else 0, np.float32)

    def shifted_blocks(x, block):
        flat = np.asarray(x).reshape(-1)
        q, _ = good_q(flat, block + 1)
        _, a = good_q(flat, block)
        return q, a

    def half_away(x, block):
        flat = np.asarray(x).reshape(-1).astype(np.float32)
        q, a = good_q(flat, block)
        s = np.repeat(np.where(a > 0, np.float32(127) / np.where(a > 0, a, 1), 0).astype(np.float32),
                      block)[:flat.size]
        v = flat * s
        return np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8), a

    def dq_no_div(q, a, block, dtype=np.float16):
        v = q.astype(np.float32) * np.repeat(a, block)[:q.size]
        with np.errstate(over="ignore"):
            return v.astype(dtype)

    def dq_next_scale(q, a, block, dtype=np.float16):
        return good_dq(q, np.roll(a, -1), block, dtype)

    def caught(qfn=None, dqfn=None):
        checks = [lambda: not _twin_mismatches(qfn, dqfn), lambda: _p17(qfn, dqfn),
                  lambda: _p18(qfn, dqfn), lambda: _p19(qfn)]
        for c in checks:
            try:
                if not c():
                    return True
            except (AssertionError, ValueError, IndexError):
                return True
        return False

    assert not caught()
    result = {"global absmax": caught(qfn=global_absmax), "shifted blocks": caught(qfn=shifted_blocks),
              "half away": caught(qfn=half_away), "no /127": caught(dqfn=dq_no_div),
              "next block's scale": caught(dqfn=dq_next_scale)}
    assert all(result.values()), result
