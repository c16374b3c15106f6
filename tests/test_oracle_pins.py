"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test names what it fixes. Sources (page title, section):
* "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models Explained",
  section 2 (outlier feature dimensions in 16-bit, the rest in int8, converted
  back to 16-bit at the end) and section 3 (threshold 6.0 on hidden states).
* "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit Depths",
  "How LLM.int8() quantizes weights and activations" (vector-wise quantization,
  outliers through a separate 16-bit product).
* "bitsandbytes: The Quantization Magic Tool for Running Large Language Models
  on Consumer Hardware", multi-level scheme, item 1 (int8 halves memory).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import brute_llmint8 as brute
import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SPECIAL = [0.0, 0.5, -0.5, 1.0, -1.0, 2.5, -2.5, 3.5, -3.5, 5.99609375, -5.99609375,
           6.0, -6.0, 127.0, -127.0]


# --------------------------------------------------------------------------- helpers

def _run_oracle(X, W, thr):
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, thr)
    return Wq, sW, st


def _near_fp16_midpoint(exact) -> bool:
    """True when an exact value lies within 1e-9 (relative) of an fp16 rounding midpoint."""
    v = float(exact)
    if v == 0.0 or not math.isfinite(v):
        return False
    a = abs(v)
    e = max(math.floor(math.log2(a)), -14)
    q = 2.0 ** (e - 10)
    frac = (a / q) % 1.0
    return abs(frac - 0.5) < 1e-9 * (a / q)


def compare_with_twin(X16, W16, thr, ora=oracle):
    """Return a list of mismatch descriptions between the oracle and the brute-force twin."""
    bad = []
    Wq, sW = ora.quantize_weight(W16)
    st = ora.linear(X16, Wq, sW, thr)
    ref = brute.forward(X16.astype(float).tolist(), W16.astype(float).tolist(), thr)
    if list(st.idx) != ref["outliers"]:
        bad.append(("outliers", list(st.idx), ref["outliers"]))
    if Wq.tolist() != ref["Wq"]:
        bad.append(("Wq",))
    if sW.astype(float).tolist() != ref["sW"]:
        bad.append(("sW",))
    if st.Xq.tolist() != ref["Xq"]:
        bad.append(("Xq", st.Xq.tolist(), ref["Xq"]))
    if st.aX.astype(float).tolist() != ref["aX"]:
        bad.append(("aX",))
    if st.C.tolist() != ref["C"]:
        bad.append(("C", st.C.tolist(), ref["C"]))
    if st.Wd.astype(float).tolist() != ref["Wd"]:
        bad.append(("Wd",))
    Y = st.Y.astype(float)
    for t in range(Y.shape[0]):
        for n in range(Y.shape[1]):
            if Y[t, n] != ref["Y"][t][n]:
                ulp_ok = _near_fp16_midpoint(ref["Y_exact"][t][n]) and \
                    abs(Y[t, n] - ref["Y"][t][n]) <= 2.0 ** (math.floor(math.log2(abs(ref["Y"][t][n]) or 1)) - 10)
                if not ulp_ok:
                    bad.append(("Y", t, n, Y[t, n], ref["Y"][t][n]))
    return bad


def _tiny_cases(seed=12345, count=300):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        T = int(rng.integers(1, 5))
        K = int(rng.integers(1, 9))
        N = int(rng.integers(1, 5))

        def draw(shape):
            a = rng.standard_normal(shape).astype(np.float32) * np.float32(rng.choice([0.05, 1.0, 4.0]))
            a = a.astype(np.float16)
            pick = rng.random(shape) < 0.45
            sp = np.array(SPECIAL, dtype=np.float16)[rng.integers(0, len(SPECIAL), size=shape)]
            a[pick] = sp[pick]
            if rng.random() < 0.15:      # an all-zero row
                a[int(rng.integers(0, shape[0]))] = 0
            return a
        X = draw((T, K))
        W = draw((N, K))
        thr = [6.0, 0.75, math.inf][i % 3]
        cases.append((X, W, thr))
    return cases


# --------------------------------------------------------------------------- P1

def test_p1_bruteforce_twin_tiny_shapes():
    """P1: every stage equals an independent pure-Python evaluation (T<=4, K<=8, N<=4)."""
    failures = []
    for X, W, thr in _tiny_cases():
        bad = compare_with_twin(X, W, thr)
        if bad:
            failures.append((X.tolist(), W.tolist(), thr, bad[:3]))
    assert not failures, failures[:3]


def test_golden_worked_example():
    """Hand-derived worked example (tests/golden/worked_example_2x4.json)."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_2x4.json")))
    X = np.array(g["X"], np.float16)
    W = np.array(g["W"], np.float16)
    Wq, sW, st = _run_oracle(X, W, g["threshold"])
    assert st.idx.tolist() == g["outliers"]
    assert Wq.tolist() == g["Wq"]
    assert sW.tolist() == g["sW"]
    assert st.Xq.tolist() == g["Xq"]
    assert st.aX.tolist() == g["aX"]
    assert st.C.tolist() == g["C"]
    assert st.Wd.astype(float).tolist() == g["Wd"]
    assert st.Y.astype(float).tolist() == g["Y"]
    # the same example through the brute-force twin
    assert not compare_with_twin(X, W, g["threshold"])


# --------------------------------------------------------------------------- P2

def _int_matrix(rng, shape):
    a = rng.integers(-127, 128, size=shape)
    for r in range(shape[0]):               # every row reaches +-127, so the scale is exactly 1
        a[r, int(rng.integers(0, shape[1]))] = 127 * (1 if rng.random() < 0.5 else -1)
    return a


@pytest.mark.parametrize("T,K,N", [(5, 40, 7), (3, 1, 2), (17, 333, 9)])
def test_p2_integer_inputs_quantize_exactly(T, K, N):
    """P2: integer X, W within +-127 (each row holding +-127), thr=inf -> Xq==X, Wq==W, C exact."""
    rng = np.random.default_rng(T * 1000 + K)
    Xi = _int_matrix(rng, (T, K))
    Wi = _int_matrix(rng, (N, K))
    Wq, sW, st = _run_oracle(Xi.astype(np.float16), Wi.astype(np.float16), math.inf)
    assert st.count == 0
    assert np.array_equal(Wq, Wi) and np.array_equal(st.Xq, Xi)
    assert np.all(sW == 127) and np.all(st.aX == 127)
    C64 = Xi.astype(np.int64) @ Wi.astype(np.int64).T          # integer routine, not BLAS
    assert np.array_equal(st.C.astype(np.int64), C64)
    # a = b = 127, so C*a*b/127**2 == C exactly and Y is C rounded once to fp16
    with np.errstate(over="ignore"):                # |C| above 65504 rounds to +-inf
        assert np.array_equal(st.Y, C64.astype(np.float64).astype(np.float16))


def test_p2_int_product_exact_at_largest_K():
    """The float64 product is exact at K=14336 with every product at the extreme 127*127."""
    rng = np.random.default_rng(7)
    K = 14336
    Xq = rng.choice(np.array([-127, 127], np.int8), size=(8, K))
    Wq = rng.choice(np.array([-127, 127], np.int8), size=(16, K))
    Wq[0] = Xq[0]                          # C[0,0] = K*127**2, the largest possible value
    C = oracle.int8_matmul(Xq, Wq)
    assert np.array_equal(C.astype(np.int64), Xq.astype(np.int64) @ Wq.astype(np.int64).T)
    assert C[0, 0] == K * 127 * 127


# --------------------------------------------------------------------------- P3

def test_p3_infinite_threshold_disables_fp16_path():
    """P3: thr=+inf (or any thr above max|X|) gives no outliers and the int8-only formula."""
    w = workloads.CONFIGS["tiny"].with_(T=16, K=256, N=64)
    W, X, cols, _ = workloads.make(w)
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, math.inf)
    assert st.count == 0 and st.Xo.shape == (16, 0) and not st.bitmap.any()
    Yint = (st.C.astype(np.float64) * st.aX[:, None] * sW[None, :] / 16129.0).astype(np.float16)
    assert np.array_equal(st.Y, Yint)
    above = float(np.abs(X.astype(np.float32)).max()) * 1.01
    st2 = oracle.linear(X, Wq, sW, above)
    assert st2.count == 0 and np.array_equal(st2.Y, st.Y) and np.array_equal(st2.Xq, st.Xq)


# --------------------------------------------------------------------------- P4

def test_p4_outlier_columns_leave_int8_path():
    """P4: Xq is zero on every outlier column; rewriting an outlier column's other
    entries (keeping one >= thr) changes neither a, Xq nor C."""
    w = workloads.CONFIGS["tiny"].with_(T=32, K=512, N=48)
    W, X, cols, _ = workloads.make(w)
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, 6.0)
    assert st.count >= len(cols) and set(cols.tolist()) <= set(st.idx.tolist())
    assert not st.Xq[:, st.idx].any()
    X2 = X.copy()
    rng = np.random.default_rng(3)
    for h in st.idx:
        keep = int(np.argmax(np.abs(X[:, h].astype(np.float32))))
        new = rng.standard_normal(X.shape[0]).astype(np.float16)
        new[keep] = X[keep, h]
        X2[:, h] = new
    st2 = oracle.linear(X2, Wq, sW, 6.0)
    assert np.array_equal(st2.idx, st.idx)
    assert np.array_equal(st2.aX, st.aX)
    assert np.array_equal(st2.Xq, st.Xq)
    assert np.array_equal(st2.C, st.C)


# --------------------------------------------------------------------------- P5

def test_p5_round_half_to_even():
    """P5: with absmax 127 the scale is 1, so halves show the rounding rule."""
    row = np.array([[127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]], np.float16)
    expect = [127, 2, 4, -2, -4, 0, 2, 0]          # half-away-from-zero would give 3, -3, 1, -1
    Wq, sW = oracle.quantize_weight(row)
    assert Wq[0].tolist() == expect and sW[0] == 127
    st = oracle.linear(row, Wq, sW, math.inf)
    assert st.Xq[0].tolist() == expect and st.aX[0] == 127


# --------------------------------------------------------------------------- P6

def test_p6_all_columns_outlier_is_plain_fp16_product():
    """P6: thr below every column's max -> C = 0 and Y = fp16(X @ Wd^T) (library matmul)."""
    rng = np.random.default_rng(11)
    X = workloads.random_fp16(rng, (9, 70), 2.0)
    X[X == 0] = np.float16(0.25)
    W = workloads.random_fp16(rng, (13, 70), 0.02)
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, 1e-3)
    assert st.count == 70 and np.all(st.aX == 0) and not st.Xq.any() and not st.C.any()
    assert np.array_equal(st.idx, np.arange(70))
    ref = np.matmul(X.astype(np.float64), st.Wd.astype(np.float64).T).astype(np.float16)
    assert np.array_equal(st.Y, ref)


# --------------------------------------------------------------------------- P7

def test_p7_zero_rows():
    """P7: an all-zero row has absmax 0, quantizes to zeros and gives an exactly zero output row."""
    w = workloads.CONFIGS["tiny"].with_(T=8, K=128, N=32)
    W, X, _, _ = workloads.make(w)
    X[3] = 0
    Wq, sW = oracle.quantize_weight(W)
    W2 = W.copy()
    W2[5] = 0
    Wq2, sW2 = oracle.quantize_weight(W2)
    assert sW2[5] == 0 and not Wq2[5].any()
    for thr in (6.0, math.inf):
        st = oracle.linear(X, Wq, sW, thr)
        assert st.aX[3] == 0 and not st.Xq[3].any()
        assert np.all(st.Y[3].astype(np.float32) == 0)


# --------------------------------------------------------------------------- P8, P9

def test_p8_outlier_set_monotone_in_threshold():
    w = workloads.CONFIGS["tiny"].with_(T=16, K=300, N=8)
    _, X, _, _ = workloads.make(w, with_weight=False)
    prev = None
    for thr in [0.5, 1.0, 2.0, 3.0, 6.0, 25.0, 70.0, math.inf]:
        m = oracle.outlier_columns(X, thr)
        if prev is not None:
            assert np.all(m <= prev)
        prev = m


def test_p9_threshold_tie_counts_as_outlier():
    """P9: an entry exactly equal to the threshold makes its column an outlier (>=)."""
    X = np.zeros((3, 40), np.float16)
    X[:] = np.float16(1.0)
    X[1, 17] = np.float16(6.0)
    assert oracle.outlier_columns(X, 6.0).nonzero()[0].tolist() == [17]
    X[1, 17] = np.float16(5.99609375)                 # the largest fp16 below 6
    assert not oracle.outlier_columns(X, 6.0).any()
    X[2, 5] = np.float16(-6.0)                        # the magnitude is what counts
    assert oracle.outlier_columns(X, 6.0).nonzero()[0].tolist() == [5]


def test_bitmap_layout():
    m = np.zeros(70, bool)
    m[[0, 31, 32, 69]] = True
    bm = oracle.pack_bitmap(m)
    assert bm.tolist() == [(1 << 0) | (1 << 31), 1, 1 << 5]


# --------------------------------------------------------------------------- P10, P11

@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (28672, 8192)])
def test_p10_memory_halves(N, K):
    """P10: int8 weight + fp32 row scale is half of fp16 plus 2/K (multi-level scheme item 1)."""
    stored = N * K * np.dtype(np.int8).itemsize + N * np.dtype(np.float32).itemsize
    ratio = stored / (N * K * np.dtype(np.float16).itemsize)
    assert ratio == pytest.approx(0.5 + 2.0 / K, rel=1e-12)
    assert ratio < 0.501


def test_p11_outlier_handling_preserves_accuracy():
    """P11: with injected large feature columns, keeping them in 16-bit gives a much
    smaller error against the exact product than quantizing them with the rest."""
    w = workloads.CONFIGS["prefill"].with_(T=64, K=1024, N=256)
    W, X, _, _ = workloads.make(w)
    Wq, sW = oracle.quantize_weight(W)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    err = {}
    for thr in (6.0, math.inf):
        Y = oracle.linear(X, Wq, sW, thr).Y.astype(np.float64)
        err[thr] = np.linalg.norm(Y - exact) / np.linalg.norm(exact)
    assert err[6.0] < 0.02
    assert err[math.inf] > 3 * err[6.0]


# --------------------------------------------------------------------------- metamorphic

def test_power_of_two_row_scaling():
    """Scaling an X row (or W row) by 2 scales its statistic by 2 and leaves the
    int8 codes and integer product unchanged (thr=inf)."""
    w = workloads.CONFIGS["tiny"].with_(T=6, K=200, N=20)
    W, X, _, _ = workloads.make(w)
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, math.inf)
    X2 = X.copy()
    X2[2] = (X2[2].astype(np.float32) * 2).astype(np.float16)
    st2 = oracle.linear(X2, Wq, sW, math.inf)
    assert np.array_equal(st2.Xq, st.Xq) and np.array_equal(st2.C, st.C)
    assert st2.aX[2] == 2 * st.aX[2]
    assert np.array_equal(st2.Y[2].astype(np.float32), 2 * st.Y[2].astype(np.float32))
    W2 = W.copy()
    W2[4] = (W2[4].astype(np.float32) / 2).astype(np.float16)
    Wq2, sW2 = oracle.quantize_weight(W2)
    assert np.array_equal(Wq2, Wq) and sW2[4] == sW[4] / 2
    st3 = oracle.linear(X, Wq2, sW2, math.inf)
    assert np.array_equal(st3.Y[:, 4].astype(np.float32), st.Y[:, 4].astype(np.float32) / 2)


def test_feature_permutation_equivariance():
    """Permuting the K axis of X and W together permutes outliers and codes and
    leaves the integer product and (up to summation order) the output unchanged;
    permuting rows of X permutes the output rows."""
    w = workloads.CONFIGS["tiny"].with_(T=12, K=96, N=24)
    W, X, _, _ = workloads.make(w)
    rng = np.random.default_rng(5)
    p = rng.permutation(96)
    Wq, sW = oracle.quantize_weight(W)
    st = oracle.linear(X, Wq, sW, 6.0)
    Wqp, sWp = oracle.quantize_weight(np.ascontiguousarray(W[:, p]))
    stp = oracle.linear(np.ascontiguousarray(X[:, p]), Wqp, sWp, 6.0)
    assert sorted(p[stp.idx].tolist()) == st.idx.tolist()
    assert np.array_equal(stp.Xq, st.Xq[:, p]) and np.array_equal(stp.aX, st.aX)
    assert np.array_equal(stp.C, st.C)
    assert oracle.parity_error(stp.Y, st.Y) <= 2.0 ** -10
    r = rng.permutation(12)
    str_ = oracle.linear(np.ascontiguousarray(X[r]), Wq, sW, 6.0)
    assert np.array_equal(str_.idx, st.idx) and np.array_equal(str_.C, st.C[r])
    assert oracle.parity_error(str_.Y, st.Y[r]) <= 2.0 ** -10


def test_parity_error_metric():
    ref = np.array([[1.0, -2.0]], np.float16)
    assert oracle.parity_error(ref, ref) == 0.0
    assert oracle.parity_error(np.array([[1.0, -2.002]], np.float16), ref) == pytest.approx(
        abs(float(np.float16(-2.002)) + 2.0) / 2.0)
    assert oracle.parity_error(np.array([[np.inf, -2.0]], np.float16), ref) == math.inf
    over = np.array([[np.inf, -np.inf, 3.0]], np.float16)      # fp16 overflow on both sides
    assert oracle.parity_error(over, over) == 0.0
    assert oracle.parity_error(np.array([[np.inf, np.inf, 3.0]], np.float16), over) == math.inf
    assert oracle.parity_error(np.array([[65504, -np.inf, 3.0]], np.float16), over) == math.inf


# --------------------------------------------------------------------------- planted mistakes

def _mutant(monkeypatch, name, fn):
    monkeypatch.setattr(oracle.llmint8_oracle, name, fn)


def _pins_fail() -> bool:
    """Run the golden example and a slice of the twin comparison against the (patched) oracle."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_2x4.json")))
    X = np.array(g["X"], np.float16)
    W = np.array(g["W"], np.float16)
    mod = oracle.llmint8_oracle
    try:
        if compare_with_twin(X, W, g["threshold"], ora=mod):
            return True
        for Xc, Wc, thr in _tiny_cases(seed=99, count=60):
            if compare_with_twin(Xc, Wc, thr, ora=mod):
                return True
        # P9 tie
        Xt = np.ones((2, 8), np.float16)
        Xt[0, 3] = 6
        if mod.outlier_columns(Xt, 6.0).sum() != 1:
            return True
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    """A plausible mistake anywhere in the oracle fails at least one pin."""
    mod = oracle.llmint8_oracle
    orig = {n: getattr(mod, n) for n in ["outlier_columns", "quantize_activations", "output",
                                          "outlier_operands", "_quantize_rows", "int8_matmul"]}
    assert not _pins_fail()

    mutants = {
        "strict threshold": ("outlier_columns",
                             lambda X, thr, *_: np.any(np.abs(X.astype(np.float32)) > np.float32(thr), axis=0)),
        "half away from zero": ("_quantize_rows", lambda v, a: (
            lambda s: np.where((a > 0)[:, None],
                               np.clip(np.sign(v * s[:, None]) * np.floor(np.abs(v * s[:, None]) + 0.5), -127, 127),
                               0).astype(np.int8))(np.where(a > 0, np.float32(127) / np.where(a > 0, a, 1), 0).astype(np.float32))),
        "outlier term dropped": ("output", lambda C, aX, sW, Xo, Wd, *r: orig["output"](C, aX, sW, Xo[:, :0], Wd[:, :0], *r)),
        "outliers kept in absmax": ("quantize_activations", lambda X, m, *_: (
            lambda q_a: (np.where(m[None, :], 0, q_a[0]).astype(np.int8), q_a[1]))(
                orig["_quantize_rows"](X.astype(np.float32), np.abs(X.astype(np.float32)).max(axis=1).astype(np.float32)))),
        "row scale ignored": ("output", lambda C, aX, sW, Xo, Wd, *r: orig["output"](
            C, np.full_like(aX, 127), sW, Xo, Wd, *r)),
        "column scale squared": ("output", lambda C, aX, sW, Xo, Wd, *r: orig["output"](
            C, aX, sW * sW, Xo, Wd, *r)),
        "dequant without /127": ("outlier_operands", lambda X, Wq, sW, idx, *_: (
            np.asarray(X)[:, idx], (Wq[:, idx].astype(np.float32) * sW[:, None]).astype(np.float16))),
        "sign flipped in product": ("int8_matmul", lambda Xq, Wq: -orig["int8_matmul"](Xq, Wq)),
    }
    caught = {}
    for label, (name, fn) in mutants.items():
        with monkeypatch.context() as m:
            m.setattr(mod, name, fn)
            caught[label] = _pins_fail()
    assert all(caught.values()), caught
