"""CPU oracle for the 4-bit weight path: blockwise NF4 / FP4 codes and the
decode-shaped linear layer that dequantizes them on the fly.

TEST INFRASTRUCTURE. Only the test-suite, the package's smoke check and the
benchmark's CPU-baseline leg import this module. The product path never does:
it shares no code, table or helper with this file (the product computes its own
code books on the host), and this file imports nothing from the product.

Sources, by page title and section:

* [DCT-4]  "bitsandbytes" (glossary), section "What it provides": the 4-bit
           layer supports a generic 4-bit float (FP4) and 4-bit NormalFloat
           (NF4), the latter fitted to the roughly normal distribution of
           trained weights; weights are quantized in blocks that each carry a
           scaling factor; the computation runs in a 16-bit type (FP16 or BF16)
           with the weights dequantized on the fly.
* [HFQ-4]  "Hugging Face Quantization with bitsandbytes ...", section 4
           "4-Bit Quantization: NF4, FP4, and Double Quantization": FP4 spreads
           its values like a generic float, NF4 puts them where normally
           distributed weights concentrate; NF4 is the default.
* [ZNX]    "bitsandbytes: The Quantization Magic Tool ...", the multi-level
           scheme list: NF4 is an information-theoretically optimized
           non-uniform 4-bit format.

Readings where the pages leave a step open:

* F1  code books (the pages give no values). NF4 follows the published
      NormalFloat construction (Dettmers et al., "QLoRA: Efficient Finetuning
      of Quantized LLMs", 2023, section 3, the technique the glossary page
      names as the one built on the library): eight positive levels at standard-normal
      quantiles Phi^-1(p) for p = p_max + i * (0.5 - p_max) / 8, i = 0..7; seven
      negative levels at -Phi^-1(p) for p = p_max + i * (0.5 - p_max) / 7,
      i = 0..6; an exact zero; everything divided by Phi^-1(p_max), with
      p_max = 1 - (1/32 + 1/30) / 2. Computed in float64, rounded once to
      fp32; code c is the c-th level in ascending order (code 7 is 0).
      FP4 is the E2M1 float: a sign bit, two exponent bits with bias 1 and one
      mantissa bit, exponent 0 subnormal; magnitudes {0, .5, 1, 1.5, 2, 3, 4,
      6}, divided by 6 so that the largest is 1; code = 8 * sign + the three
      magnitude bits (code 8 is -0).
* F2  blocks are ``block`` consecutive elements of the flat row-major weight
      (the last one may be shorter); each keeps its absolute maximum ``a`` in
      fp32 (exact: the inputs are 16-bit).
* F3  codes: ``x_n = fl32(w / a)`` (``x_n = 0`` when ``a = 0``); the code is
      that of the level nearest to ``x_n``, decided against the fp32 midpoints
      ``fl32(fl32(l_i + l_{i+1}) * 0.5)`` of adjacent distinct levels in
      ascending order: the rank is the number of midpoints strictly below
      ``x_n``, so a value equal to a midpoint takes the lower level. For FP4
      the zero is the +0 code.
* F4  two codes per byte, the element with the even flat index in the low
      nibble.
* F5  dequantization: ``Wdeq = r16(fl32(c[code] * a))``, rounded to the 16-bit
      compute type (fp16, or bf16 as bit patterns).
* F6  linear: ``Y = r16(X . Wdeq^T + bias)``: 16-bit operands, a wide sum
      (float64 here), one rounding to the compute type.
"""
from __future__ import annotations

import numpy as np

from .llmint8_oracle import _to_f32, f32_to_bf16_bits, f64_to_bf16_bits

__all__ = ["NF4_P_MAX", "code_book", "quantize_levels", "quantize_4bit", "unpack_4bit",
           "dequantize_4bit", "linear_4bit"]

NF4_P_MAX = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def code_book(quant_type: str) -> np.ndarray:
    """fp32 value of each 4-bit code, indexed by code (F1)."""
    if quant_type == "nf4":
        from scipy.stats import norm
        d = norm.ppf(NF4_P_MAX)
        step_pos = (0.5 - NF4_P_MAX) / 8.0
        step_neg = (0.5 - NF4_P_MAX) / 7.0
        pos = [norm.ppf(NF4_P_MAX + i * step_pos) / d for i in range(8)]
        neg = [-norm.ppf(NF4_P_MAX + i * step_neg) / d for i in range(7)]
        return np.array(sorted(neg + [0.0] + pos), dtype=np.float64).astype(np.float32)
    if quant_type == "fp4":
        vals = np.zeros(16, dtype=np.float64)
        for code in range(16):
            sign, e, m = code >> 3, (code >> 1) & 3, code & 1
            mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
            vals[code] = -mag / 6.0 if sign else mag / 6.0
        return vals.astype(np.float32)
    raise ValueError(f"unknown 4-bit type {quant_type!r}")


def quantize_levels(quant_type: str):
    """(codes of the distinct levels in ascending order, fp32 midpoints between them) (F3)."""
    book = code_book(quant_type)
    codes = [c for c in range(16) if not (book[c] == 0 and np.signbit(book[c]))]
    order = np.array(sorted(codes, key=lambda c: float(book[c])), dtype=np.int64)
    lev = book[order]
    mids = (lev[:-1] + lev[1:]) * np.float32(0.5)
    return order, mids.astype(np.float32)


def quantize_4bit(W16: np.ndarray, block: int, quant_type: str, dtype: str = "f16"):
    """Blockwise 4-bit quantization of a 16-bit tensor taken flat (F2-F4).

    Returns ``(packed uint8[ceil(n / 2)], absmax fp32[ceil(n / block)])``.
    """
    v32 = _to_f32(np.asarray(W16).reshape(-1), dtype)
    n = v32.shape[0]
    nb = -(-n // block)
    blocks = np.concatenate([v32, np.zeros(nb * block - n, np.float32)]).reshape(nb, block)
    a = np.max(np.abs(blocks), axis=1).astype(np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    xn = np.where(a[:, None] > 0, blocks / safe[:, None], np.float32(0.0)).astype(np.float32)
    order, mids = quantize_levels(quant_type)
    rank = np.searchsorted(mids, xn.reshape(-1), side="left")
    codes = order[rank][:n].astype(np.uint8)
    if n % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    packed = (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8)
    return packed, a


def unpack_4bit(packed: np.ndarray, n: int) -> np.ndarray:
    """Codes of elements 0..n-1 (F4)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    codes = np.empty(2 * p.shape[0], dtype=np.uint8)
    codes[0::2] = p & np.uint8(15)
    codes[1::2] = p >> np.uint8(4)
    return codes[:n]


def dequantize_4bit(packed: np.ndarray, absmax: np.ndarray, block: int, quant_type: str, n: int,
                    dtype: str = "f16") -> np.ndarray:
    """``r16(fl32(c[code] * a))`` for elements 0..n-1 (F5); fp16 values, or bf16 bit patterns."""
    book = code_book(quant_type)
    c = book[unpack_4bit(packed, n)]
    a = np.repeat(np.asarray(absmax, dtype=np.float32), block)[:n]
    v = (c * a).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    return v.astype(np.float16)


def linear_4bit(X16: np.ndarray, packed: np.ndarray, absmax: np.ndarray, block: int,
                quant_type: str, N: int, dtype: str = "f16",
                bias: np.ndarray | None = None) -> np.ndarray:
    """``Y = r16(X . Wdeq^T + bias)`` with the weight dequantized per call (F5, F6).

    ``X16`` is [T, K] in the compute type; the weight is [N, K] in flat
    row-major order. The 16-bit products are exact in float64 and the sum is
    formed in float64 before the single rounding.
    """
    X = np.asarray(X16)
    K = X.shape[1]
    Wd = dequantize_4bit(packed, absmax, block, quant_type, N * K, dtype).reshape(N, K)
    Y64 = _to_f32(X, dtype).astype(np.float64) @ _to_f32(Wd, dtype).astype(np.float64).T
    if bias is not None:
        Y64 = Y64 + _to_f32(np.asarray(bias), dtype).astype(np.float64)[None, :]
    if dtype == "bf16":
        return f64_to_bf16_bits(Y64)
    with np.errstate(over="ignore"):
        return Y64.astype(np.float16)
