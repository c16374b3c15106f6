"""CPU oracle for the LLM.int8() mixed-precision decomposition linear layer.

TEST INFRASTRUCTURE. Only the test-suite, the package's smoke check and the
benchmark's CPU-baseline leg import this module. The product path never does:
it shares no code, table or helper with this file, and this file imports
nothing from the product.

What it computes, stage by stage, in the order the method takes them. Sources
are cited by page title and section:

* [HFQ-2]  "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
           Explained", section 2 "LLM.int8(): Quantizing Without Degrading
           Large Models": outliers are whole feature dimensions of large
           magnitude; they are computed in 16-bit while the rest is multiplied
           in int8 and converted back to 16-bit at the end.
* [HFQ-3]  same page, section 3 "Configuring 8-Bit Loading": the outlier
           cutoff ``llm_int8_threshold``, default 6.0, applies to hidden-state
           (activation) values.
* [HYS]    "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit
           Depths", section "How LLM.int8() quantizes weights and activations":
           vector-wise quantization; values that fit 8-bit are quantized,
           outliers go through a separate 16-bit matrix multiplication.
* [HEAT]   "Shrink LLMs to 4-bit and train them anyway", section "The
           interesting bit": vector-wise quantization for the bulk, outliers
           through 16-bit matmul.
* [DCT]    "bitsandbytes" (mining glossary), sections "What it provides" (the
           large *activation* values are kept in higher precision) and the
           introduction (weights are quantized when the model loads).

Readings where the pages leave a step open:

* R1  an outlier is a whole *column* (feature dimension) of X, decided over all
      T rows of the call; the weight has no threshold.
* R2  a column is an outlier when some |x| *reaches* the threshold (``>=``).
* R3  the row statistic of X is the absolute maximum over the non-outlier
      columns only.
* R4  absmax ("vector-wise") scaling: ``s = fl32(127 / absmax)`` computed once
      per row, ``q = rne(fl32(v * s))``; symmetric, so -128 never occurs.
* R5  a row whose absmax is 0 quantizes to all zeros and keeps scale 0.
* R6  the weight is quantized once per output row over all K.
* R7  the 16-bit weight operand of the outlier product is the stored int8
      weight dequantized: ``fp16(fl32(fl32(q * b) / 127))``.
* R8  the outlier product has fp16 operands; the output is rounded once to fp16.
* R9  the threshold is compared in fp32; ``+inf`` gives an empty outlier set.
* B1  the input gradient through the frozen layer, used to train an adapter on
      top of it, treats the layer as the linear map ``X -> X . Wdeq^T`` with the
      stored weight dequantized per operation, ``Wdeq = fp16(fl32(fl32(q * b) /
      127))`` for every entry (as in R7); quantizing X has no useful derivative.
      ``dX = fp16(dY . Wdeq)``: fp16 operands, a wide accumulation, one
      rounding to fp16. With bf16 activations (B2) dY, Wdeq and dX are bf16.

* B2  bf16 activations: with ``dtype="bf16"`` X, the bias and Y are bfloat16
      (carried here as uint16 bit patterns). Every bf16 value is exact in
      fp32, so the outlier test and the quantization are the same fp32
      operations as for fp16; the outlier operand ``Wd`` is rounded to bf16
      and the 16-bit product takes bf16 operands; Y is rounded once to bf16
      (round to nearest even).
* B3  bias: an optional vector [N] in the activation dtype, added to the sum
      before the single final rounding.
* Q1  blockwise 8-bit codec: a flat tensor is cut into blocks of ``block``
      consecutive elements (the last one may be shorter); each block keeps its
      absolute maximum ``a`` (fp32) and codes ``q = rne(fl32(x * fl32(127 / a)))``
      (the R4 rule per block; a zero block gives codes 0 and a = 0).
      Dequantization is ``fl32(fl32(q * a) / 127)`` (the R7 form), returned in
      the input's dtype (fp16 rounds once more). The pages give neither the
      block size nor a code table: the block size is the caller's, and the
      code is the same symmetric linear one as the rest of the method.

The bf16 and bias sources:

* [HFQ-5]  "Hugging Face Quantization with bitsandbytes ...", section 5
           "Storage Precision vs. Compute Precision": the storage type of the
           weights and the compute type (bfloat16 preferred where the hardware
           has it, else float16) are separate choices.
* [HYS-L]  "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit
           Depths": ``Linear8bitLt`` is a drop-in replacement for a linear
           layer (which carries a bias).

The backward sources:

* [HFQ-T]  "Hugging Face Quantization with bitsandbytes ...", the quick
           comparison table before section 1 (an int8 model is not trained
           directly: it is frozen and an adapter is added) and section 6
           "Quantization for Inference vs. Quantization for Training (QLoRA)"
           (the quantized weights stay frozen while gradients still have to
           flow through them).
* [DCT-S]  "bitsandbytes" (mining glossary), "Where it fits in the stack":
           weights are dequantized for each operation instead of being
           computed on directly.

The blockwise codec sources:

* [DCT-P]  "bitsandbytes" (mining glossary), "What it provides": weights are
           quantized in blocks, each with its own scaling factor, so that one
           outlier only affects its own block.
* [HYS-O]  "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit
           Depths", the 8-bit optimizers: block-wise quantization shrinks the
           optimizer states.

Precision: every quantization step is the fp32 operation named (NumPy float32
arithmetic is IEEE round-to-nearest-even); ``np.rint`` is round-half-to-even.
The integer product is a float64 matrix product of the int8 values, which is
exact because every partial sum is an integer of magnitude below 2**31 < 2**53.
The output is formed in float64 and rounded once to fp16.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "quantize_weight", "outlier_columns", "pack_bitmap", "quantize_activations",
    "int8_matmul", "outlier_operands", "output", "linear", "Stages", "parity_error",
    "dequantize_weight", "linear_backward_input", "quantize_blockwise", "dequantize_blockwise",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "f64_to_bf16_bits",
]

_F32_127 = np.float32(127.0)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def f64_to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns with one rounding to 8 significant bits,
    nearest even (finite inputs; beyond the bf16 range gives +-inf)."""
    x = np.asarray(x64, dtype=np.float64)
    m, e = np.frexp(x)                               # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                          # bf16 subnormals share the 2**-133 quantum
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)  # 8 significant bits, half to even
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)                   # exact unless beyond fp32 range (-> inf)
    big = np.abs(r) > float(np.float32(3.3895313892515355e38))
    r32 = np.where(big, np.copysign(np.float32(np.inf), r32), r32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _to_f32(A, dtype: str) -> np.ndarray:
    """Activation-dtype array (fp16 values, or bf16 bit patterns) -> exact fp32."""
    A = np.asarray(A)
    if dtype == "bf16":
        assert A.dtype == np.uint16
        return bf16_bits_to_f32(A)
    assert dtype == "f16" and A.dtype == np.float16
    return A.astype(np.float32)


def _to_f64(A, dtype: str) -> np.ndarray:
    return _to_f32(A, dtype).astype(np.float64)


def _absmax_rows(v32: np.ndarray) -> np.ndarray:
    if v32.shape[1] == 0:
        return np.zeros(v32.shape[0], np.float32)
    return np.abs(v32).max(axis=1).astype(np.float32)


def _quantize_rows(v32: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """R4/R5: q = rne(fl32(v * fl32(127/absmax))) per row, 0 where absmax == 0."""
    pos = absmax > 0
    s = np.zeros_like(absmax)
    s[pos] = _F32_127 / absmax[pos]                 # fp32 correctly-rounded division
    prod = v32 * s[:, None]                         # fp32 multiply
    q = np.rint(prod)                               # round half to even
    q = np.clip(q, -127, 127)                       # no-op for |v| <= absmax
    q[~pos, :] = 0
    return q.astype(np.int8)


def quantize_weight(W16: np.ndarray, dtype: str = "f16"):
    """Vector-wise weight quantization at load time ([HYS]; [DCT] introduction; R4-R6).

    ``W16`` fp16 [N, K] (or bf16 bit patterns with ``dtype="bf16"``) ->
    (``Wq`` int8 [N, K], ``sW`` fp32 [N]) with ``sW[n] = max_k |W[n, k]|``
    (exact: a 16-bit value) and ``Wq[n, k] = rne(fl32(W[n, k] * fl32(127 / sW[n])))``.
    """
    W = np.asarray(W16)
    assert W.ndim == 2
    W32 = _to_f32(W, dtype)
    b = _absmax_rows(W32)
    return _quantize_rows(W32, b), b


def outlier_columns(X16: np.ndarray, threshold: float, dtype: str = "f16") -> np.ndarray:
    """Outlier feature dimensions ([HFQ-2]; [HFQ-3]; R1, R2, R9).

    Returns a bool mask [K]: column h is an outlier when some row has
    ``|X[t, h]| >= threshold`` (fp32 comparison).
    """
    X = np.asarray(X16)
    assert X.ndim == 2
    thr = np.float32(threshold)
    return np.any(np.abs(_to_f32(X, dtype)) >= thr, axis=0)


def pack_bitmap(mask: np.ndarray) -> np.ndarray:
    """Bitmap form of the outlier set: bit (h % 32) of uint32 word h // 32 is column h."""
    K = mask.shape[0]
    words = np.zeros((K + 31) // 32, np.uint32)
    for h in np.flatnonzero(mask):
        words[h // 32] |= np.uint32(1) << np.uint32(h % 32)
    return words


def quantize_activations(X16: np.ndarray, outlier_mask: np.ndarray, dtype: str = "f16"):
    """Row-wise (vector-wise) quantization of the non-outlier part of X ([HYS]; R3-R5).

    ``a[t] = max over non-outlier columns of |X[t, k]|``;
    ``Xq[t, k] = 0`` on outlier columns, else ``rne(fl32(X[t, k] * fl32(127 / a[t])))``.
    """
    X32 = _to_f32(X16, dtype)
    kept = np.where(outlier_mask[None, :], np.float32(0), X32)
    a = _absmax_rows(kept)
    return _quantize_rows(kept, a), a


def int8_matmul(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """The int8 product with integer accumulation ([HFQ-2]: "multiplied in int8").

    ``C = Xq @ Wq.T`` exactly, returned as int32.
    """
    C = Xq.astype(np.float64) @ Wq.astype(np.float64).T
    Ci = C.astype(np.int64)
    assert np.all(Ci == C), "float64 product of int8 values must be exact"
    assert Ci.size == 0 or np.abs(Ci).max() < 2 ** 31
    return Ci.astype(np.int32)


def outlier_operands(X16: np.ndarray, Wq: np.ndarray, sW: np.ndarray, idx: np.ndarray,
                     dtype: str = "f16"):
    """16-bit operands of the outlier product ([HYS]; [HFQ-2]; R7, R8, B2).

    ``Xo = X[:, idx]`` (exact copy, activation dtype);
    ``Wd[n, j] = r16(fl32(fl32(Wq[n, idx[j]] * sW[n]) / 127))`` with r16 the
    rounding to the activation dtype.
    """
    Xo = np.asarray(X16)[:, idx]
    q32 = Wq[:, idx].astype(np.float32)
    d32 = (q32 * sW[:, None].astype(np.float32)) / _F32_127
    Wd = f32_to_bf16_bits(d32) if dtype == "bf16" else d32.astype(np.float16)
    return Xo, Wd


def output(C: np.ndarray, aX: np.ndarray, sW: np.ndarray, Xo: np.ndarray, Wd: np.ndarray,
           dtype: str = "f16", bias: np.ndarray | None = None):
    """Recombination, converted back to 16-bit at the end ([HFQ-2]; B2, B3).

    ``Y = r16( C * a[t] * b[n] / 127**2  +  Xo @ Wd.T  +  bias[n] )`` evaluated
    in float64 and rounded once to the activation dtype.
    """
    Y64 = C.astype(np.float64) * aX.astype(np.float64)[:, None] \
        * sW.astype(np.float64)[None, :] / 16129.0
    if Xo.shape[1]:
        Y64 = Y64 + _to_f64(Xo, dtype) @ _to_f64(Wd, dtype).T
    if bias is not None:
        Y64 = Y64 + _to_f64(bias, dtype)[None, :]
    if dtype == "bf16":
        return f64_to_bf16_bits(Y64)
    with np.errstate(over="ignore"):               # beyond fp16 range: +-inf, like any fp16 cast
        return Y64.astype(np.float16)


@dataclasses.dataclass
class Stages:
    outlier_mask: np.ndarray   # bool [K]
    bitmap: np.ndarray         # uint32 [ceil(K/32)]
    idx: np.ndarray            # int32 [|O|], ascending
    Xq: np.ndarray             # int8 [T, K]
    aX: np.ndarray             # fp32 [T]
    C: np.ndarray | None       # int32 [T, N] (None when rows were restricted)
    Xo: np.ndarray             # fp16 [T, |O|]
    Wd: np.ndarray             # fp16 [N, |O|]
    Y: np.ndarray | None       # fp16 [T, N]

    @property
    def count(self) -> int:
        return int(self.idx.shape[0])


def linear(X16: np.ndarray, Wq: np.ndarray, sW: np.ndarray, threshold: float,
           rows: np.ndarray | None = None, with_outputs: bool = True, dtype: str = "f16",
           bias: np.ndarray | None = None) -> Stages:
    """The whole forward: outlier set, quantized activations, int8 product, output.

    ``rows`` restricts C and Y to a subset of rows (the outlier set and row
    statistics are still taken over all of X, as the method defines them).
    ``dtype`` is the activation type ("f16", or "bf16" with X, bias and Y as
    bf16 bit patterns); ``bias`` an optional [N] vector of that type.
    """
    mask = outlier_columns(X16, threshold, dtype)
    idx = np.flatnonzero(mask).astype(np.int32)
    Xq, aX = quantize_activations(X16, mask, dtype)
    Xo, Wd = outlier_operands(X16, Wq, sW, idx, dtype)
    C = Y = None
    if with_outputs:
        sel = slice(None) if rows is None else rows
        C = int8_matmul(Xq[sel], Wq)
        Y = output(C, aX[sel], sW, Xo[sel], Wd, dtype, bias)
    return Stages(mask, pack_bitmap(mask), idx, Xq, aX, C, Xo, Wd, Y)


def parity_error(Y_test: np.ndarray, Y_ref: np.ndarray) -> float:
    """Max-abs error normalised by the reference's max-abs finite value (floor 2**-14).

    Entries where the reference overflowed fp16 (+-inf) must match exactly; any
    other non-finite test value is an infinite error.
    """
    a = Y_test.astype(np.float64)
    r = Y_ref.astype(np.float64)
    if r.size == 0:
        return 0.0
    fin = np.isfinite(r)
    if np.any(a[~fin] != r[~fin]) or not np.all(np.isfinite(a[fin])):
        return float("inf")
    if not fin.any():
        return 0.0
    den = max(float(np.abs(r[fin]).max()), 2.0 ** -14)
    return float(np.abs(a[fin] - r[fin]).max() / den)


def dequantize_weight(Wq: np.ndarray, sW: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """The stored weight dequantized per operation ([DCT-S]; R7, B1, B2).

    ``Wdeq[n, k] = r16(fl32(fl32(Wq[n, k] * sW[n]) / 127))`` for every entry,
    ``r16`` the rounding to fp16 (or, with ``dtype="bf16"``, to bf16 bit
    patterns); the outlier operand ``Wd`` of the forward is its columns at the
    outliers.
    """
    q32 = np.asarray(Wq).astype(np.float32)
    d32 = (q32 * np.asarray(sW, dtype=np.float32)[:, None]) / _F32_127
    if dtype == "bf16":
        return f32_to_bf16_bits(d32)
    return d32.astype(np.float16)


def linear_backward_input(dY16: np.ndarray, Wq: np.ndarray, sW: np.ndarray,
                          dtype: str = "f16") -> np.ndarray:
    """Input gradient of the frozen layer, the step that lets an adapter train on top of it ([HFQ-T]; B1).

    ``dX = r16( dY @ Wdeq )`` with ``Wdeq = dequantize_weight(Wq, sW, dtype)``:
    the 16-bit products are exact in float64, the sum is formed in float64 and
    the result is rounded once to the 16-bit type (fp16, or bf16 as bit
    patterns with ``dtype="bf16"``, where dY is bf16 bit patterns too: B2).
    """
    Wd = dequantize_weight(Wq, sW, dtype)
    dX64 = _to_f64(np.asarray(dY16), dtype) @ _to_f64(Wd, dtype)
    if dtype == "bf16":
        return f64_to_bf16_bits(dX64)
    with np.errstate(over="ignore"):
        return dX64.astype(np.float16)


def quantize_blockwise(x: np.ndarray, block: int):
    """Blockwise absmax int8 quantization of a flat tensor ([DCT-P], [HYS-O]; Q1).

    ``x`` is fp16 or fp32 (any shape, taken flat). Returns ``(q int8[n],
    absmax fp32[ceil(n / block)])``; block ``b`` covers elements
    ``[b * block, min((b + 1) * block, n))``.
    """
    flat = np.asarray(x).reshape(-1)
    n = flat.shape[0]
    nb = -(-n // block)
    v32 = flat.astype(np.float32)
    pad = nb * block - n
    blocks = np.concatenate([v32, np.zeros(pad, np.float32)]).reshape(nb, block)
    a = _absmax_rows(blocks)
    q = _quantize_rows(blocks, a).reshape(-1)[:n]
    return q.astype(np.int8), a


def dequantize_blockwise(q: np.ndarray, absmax: np.ndarray, block: int, dtype=np.float16):
    """Inverse of ``quantize_blockwise`` (Q1): ``fl32(fl32(q * a) / 127)``, then
    rounded to ``dtype`` (fp16 or fp32)."""
    q32 = np.asarray(q).reshape(-1).astype(np.float32)
    n = q32.shape[0]
    a = np.repeat(np.asarray(absmax, dtype=np.float32), block)[:n]
    v = (q32 * a) / _F32_127
    return v.astype(dtype)
