"""Independent brute-force twin of the LLM.int8() forward, for tiny inputs.

Pure Python: loops, Python ``int`` for the integer product, ``fractions.Fraction``
for the exact output value, ``struct`` for IEEE rounding to fp32 / fp16. It uses
no NumPy and nothing from the oracle, so agreement between the two pins the
oracle's vectorised arithmetic (indices, operand order, scales, rounding).

Rounding facts it relies on:
* ``struct.pack('f', x)`` rounds a binary64 value to the nearest fp32 (ties to
  even); ``struct.pack('e', x)`` does the same to fp16.
* An fp16 value times an fp32 value, or a 7-bit integer times an fp32 value, is
  exact in binary64 (at most 35 and 31 significant bits), so one rounding to
  fp32 afterwards is the IEEE fp32 product.
* A binary64 quotient of two fp32 values, rounded again to fp32, is the
  correctly-rounded fp32 quotient (53 >= 2*24 + 2).
* Python's ``round()`` on a float rounds half to even.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f16(x: float) -> float:
    return struct.unpack("<e", struct.pack("<e", x))[0]


def f16_of_fraction(q: Fraction) -> float:
    """Correct round-half-even of an exact rational to fp16 (finite range only)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix possible off-by-one of the float log
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                      # subnormal range shares the 2**-24 quantum
    quantum = Fraction(2) ** (e - 10)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * quantum
    if val > 65504:
        return sign * math.inf
    return sign * float(val)


def bf16_of_fraction(q: Fraction) -> float:
    """Correct round-half-even of an exact rational to bfloat16 (8 significant
    bits, the fp32 exponent range; finite results only)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # subnormals share the 2**-133 quantum
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * quantum)


def bf16(x: float) -> float:
    return bf16_of_fraction(Fraction(x))


def rne(x: float) -> int:
    return int(round(x))


def quantize_vector(vals):
    """absmax row quantization; returns (q list, absmax)."""
    m = 0.0
    for v in vals:
        m = max(m, abs(v))
    if m == 0.0:
        return [0] * len(vals), 0.0
    s = f32(127.0 / m)
    q = []
    for v in vals:
        r = rne(f32(v * s))
        q.append(max(-127, min(127, r)))
    return q, m


def forward(X, W, thr, bf16_io=False, bias=None):
    """X: T x K list of fp16-valued floats (bf16-valued with ``bf16_io``);
    W: N x K; thr: float; bias: optional list of N 16-bit values.

    Returns dict with outlier list, Wq, sW, Xq, aX, C, Y (Y as floats).
    """
    r16 = bf16 if bf16_io else f16
    r16_exact = bf16_of_fraction if bf16_io else f16_of_fraction
    T = len(X)
    N = len(W)
    K = len(W[0]) if N else (len(X[0]) if T else 0)
    thr32 = f32(thr) if math.isfinite(thr) else thr
    outl = []
    for h in range(K):
        hit = False
        for t in range(T):
            if abs(X[t][h]) >= thr32:
                hit = True
        if hit:
            outl.append(h)
    oset = set(outl)
    Wq, sW = [], []
    for n in range(N):
        q, b = quantize_vector(W[n])
        Wq.append(q)
        sW.append(b)
    Xq, aX = [], []
    for t in range(T):
        kept = [0.0 if h in oset else X[t][h] for h in range(K)]
        q, a = quantize_vector(kept)
        Xq.append(q)
        aX.append(a)
    C = [[sum(Xq[t][k] * Wq[n][k] for k in range(K)) for n in range(N)] for t in range(T)]
    Wd = [[r16(f32(f32(Wq[n][h] * sW[n]) / 127.0)) for h in outl] for n in range(N)]
    Y = []
    for t in range(T):
        row = []
        for n in range(N):
            exact = Fraction(C[t][n]) * Fraction(aX[t]) * Fraction(sW[n]) / 16129
            for j, h in enumerate(outl):
                exact += Fraction(X[t][h]) * Fraction(Wd[n][j])
            if bias is not None:
                exact += Fraction(bias[n])
            row.append((exact, r16_exact(exact)))
        Y.append(row)
    return {"outliers": outl, "Wq": Wq, "sW": sW, "Xq": Xq, "aX": aX, "C": C, "Wd": Wd,
            "Y": [[y for _, y in r] for r in Y], "Y_exact": [[e for e, _ in r] for r in Y]}


def backward_input(dY, Wq, sW, to_bf16=False):
    """Input gradient through the frozen layer, for tiny inputs.

    dY: T x N list of fp16-valued (bf16-valued with ``to_bf16``) floats; Wq:
    N x K list of ints; sW: N floats. Each dequantized entry is
    r16(fl32(fl32(q * b) / 127)) (fp32 product and quotient by the rounding
    facts above); the sum over n of dY * Wdeq is an exact Fraction, rounded
    once to the 16-bit type.
    """
    r16 = bf16 if to_bf16 else f16
    r16_exact = bf16_of_fraction if to_bf16 else f16_of_fraction
    T = len(dY)
    N = len(Wq)
    K = len(Wq[0]) if N else 0
    Wdeq = [[r16(f32(f32(Wq[n][k] * sW[n]) / 127.0)) for k in range(K)] for n in range(N)]
    dX = []
    for t in range(T):
        row = []
        for k in range(K):
            acc = Fraction(0)
            for n in range(N):
                acc += Fraction(dY[t][n]) * Fraction(Wdeq[n][k])
            row.append(r16_exact(acc))
        dX.append(row)
    return Wdeq, dX


def quantize_blockwise(vals, block):
    """Blockwise absmax codes of a flat list of fp16- or fp32-valued floats."""
    q, absmax = [], []
    for b0 in range(0, len(vals), block):
        codes, m = quantize_vector(vals[b0:b0 + block])
        q.extend(codes)
        absmax.append(m)
    return q, absmax


def dequantize_blockwise(q, absmax, block, to_fp16):
    out = []
    for i, c in enumerate(q):
        v = f32(f32(c * absmax[i // block]) / 127.0)
        out.append(f16(v) if to_fp16 else v)
    return out


# --------------------------------------------------------------------------- 4-bit weight path

NF4_P_MAX = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def phi(x: float) -> float:
    """Standard normal CDF from math.erfc."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def normal_quantile(p: float) -> float:
    """Phi^-1(p) by bisection on ``phi`` (no library inverse)."""
    lo, hi = -12.0, 12.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid in (lo, hi):
            break
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def nf4_book():
    """NF4 levels by code: normal quantiles on two evenly spaced probability
    grids (8 positive, 7 negative) plus zero, scaled so the largest is 1."""
    d = normal_quantile(NF4_P_MAX)
    pos = [normal_quantile(NF4_P_MAX + i * ((0.5 - NF4_P_MAX) / 8.0)) / d for i in range(8)]
    neg = [-normal_quantile(NF4_P_MAX + i * ((0.5 - NF4_P_MAX) / 7.0)) / d for i in range(7)]
    return [f32(v) for v in sorted(neg + [0.0] + pos)]


def fp4_book():
    """FP4 (E2M1) levels by code, decoded through an fp32 bit pattern, then / 6."""
    out = []
    for code in range(16):
        sign, e, m = code >> 3, (code >> 1) & 3, code & 1
        if e == 0 and m == 0:
            bits = sign << 31
        elif e == 0:
            bits = (sign << 31) | (126 << 23)               # subnormal 0.5
        else:
            bits = (sign << 31) | ((e - 1 + 127) << 23) | (m << 22)
        v = struct.unpack("<f", struct.pack("<I", bits))[0]
        out.append(f32(v / 6.0))
    return out


def _levels(book):
    """(level value, code) pairs of the distinct levels, ascending; -0 dropped."""
    pairs = [(v, c) for c, v in enumerate(book) if not (v == 0.0 and math.copysign(1.0, v) < 0)]
    return sorted(pairs)


def quantize_4bit(vals, block, book):
    """Blockwise 4-bit codes of a flat list of 16-bit-valued floats; packed bytes, absmax."""
    lev = _levels(book)
    mids = [f32(f32(lev[i][0] + lev[i + 1][0]) * 0.5) for i in range(len(lev) - 1)]
    codes, absmax = [], []
    for b0 in range(0, len(vals), block):
        blk = vals[b0:b0 + block]
        a = 0.0
        for v in blk:
            a = max(a, abs(v))
        absmax.append(a)
        for v in blk:
            xn = f32(v / a) if a > 0 else 0.0
            rank = 0
            for m in mids:
                if m < xn:
                    rank += 1
            codes.append(lev[rank][1])
    if len(codes) % 2:
        codes.append(0)
    packed = [codes[i] | (codes[i + 1] << 4) for i in range(0, len(codes), 2)]
    return packed, absmax


def dequantize_4bit(packed, absmax, block, book, n, to_bf16=False):
    out = []
    for i in range(n):
        code = (packed[i // 2] >> (4 * (i % 2))) & 15
        v = f32(book[code] * absmax[i // block])
        out.append(bf16(v) if to_bf16 else f16(v))
    return out


def linear_4bit(X, packed, absmax, block, book, N, to_bf16=False, bias=None):
    """Y[t][n] = r16(sum_k X[t][k] * Wdeq[n][k] + bias[n]), exact sum, one rounding."""
    K = len(X[0])
    Wd = dequantize_4bit(packed, absmax, block, book, N * K, to_bf16)
    r = bf16_of_fraction if to_bf16 else f16_of_fraction
    Y = []
    for row in X:
        out = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(row[k]) * Fraction(Wd[n * K + k])
            if bias is not None:
                acc += Fraction(bias[n])
            out.append(r(acc))
        Y.append(out)
    return Y
