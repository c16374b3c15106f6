"""Seeded synthetic inputs for the LLM.int8() linear layer.

This module only draws random numbers and places them: it holds none of the
method's arithmetic (no quantization, no outlier test, no product), so both the
CPU oracle and the GPU path can be fed from it without sharing any of the
computation.

The value distributions follow the workloads the method is about ("Hugging Face
Quantization with bitsandbytes", section 2: a few feature dimensions carry
values far larger than the rest): activations are standard normal, a handful of
whole feature columns are replaced by large-magnitude values, and weights are a
small-variance normal matrix.

Recipe. The weight comes from ``Generator(PCG64(SeedSequence([seed, 0])))``
and the activations from ``Generator(PCG64(SeedSequence([seed, 1])))``, each in
the draw order below, so either can be drawn without the other:

1. ``W = fp16(sigma * standard_normal((N, K), float32))``
2. ``cols = sort(choice(K, n_out, replace=False))``
3. ``Z = standard_normal((T, K), float32)``; ``X = fp16(Z)``; then for every
   injected column ``X[:, cols] = fp16(sign(Z[:, cols]) * uniform(lo, hi))``,
   with ``sign(0) = +1`` and the uniform draws float32 of shape ``(T, n_out)``.
4. (only when ``zero_rows > 0``) ``rows = sort(choice(T, zero_rows,
   replace=False))``; ``X[rows[:, None], cols[None, :]] = 0``.

5. (input-gradient checks only) the output gradient comes from
   ``Generator(PCG64(SeedSequence([seed, 2])))``:
   ``dY = fp16(standard_normal((T, N), float32))``.

6. (blockwise codec only) an fp32 tensor shaped like an optimizer state comes
   from ``Generator(PCG64(SeedSequence([seed, 3])))``:
   ``s = float32(1e-3 * standard_normal(n))``, then every 1000th element times
   50 (isolated large values, one per few blocks).

7. (bf16 checks only) bf16 inputs are the fp16 draws above widened to float32
   and cut to their upper 16 bits (truncation toward zero, so every value is
   an exact bf16 and the injected columns keep their magnitudes to 1%).

8. (bias checks only) a bias vector comes from
   ``Generator(PCG64(SeedSequence([seed, 4])))``:
   ``bias = float32(0.5 * standard_normal(N))``, stored as fp16, or as bf16 by
   the truncation of step 7.

Natural N(0,1) entries can still cross the threshold on their own; the set of
outlier columns is always whatever the method computes, not ``cols``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_weight", "make_activations", "make", "make_output_grad",
           "make_state", "as_bf16_input", "make_bias"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    K: int
    N: int
    sigma: float           # std-dev of the weight entries
    n_out: int             # injected large-magnitude feature columns
    lo: float              # |x| of injected entries ~ U(lo, hi)
    hi: float
    threshold: float
    seed: int
    zero_rows: int = 0     # rows whose injected entries are zeroed afterwards

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _cfg4_zero_rows(T: int) -> int:
    return int(math.ceil(0.01 * T))


# The five workload shapes this library is measured and checked on.
CONFIGS = {
    # tiny: latency-bound, parity only
    "tiny": Workload("tiny", T=16, K=1024, N=1024, sigma=0.02, n_out=4, lo=20.0, hi=60.0,
                     threshold=6.0, seed=1),
    # decode-shaped GEMV; T=1 and T=4 use the first rows of the T=8 draw
    "decode": Workload("decode", T=8, K=4096, N=4096, sigma=0.02, n_out=6, lo=20.0, hi=60.0,
                       threshold=6.0, seed=2),
    # prefill MLP up-projection
    "prefill": Workload("prefill", T=2048, K=4096, N=11008, sigma=0.02, n_out=6, lo=20.0,
                        hi=60.0, threshold=6.0, seed=3),
    # large hidden size MLP, 1% of rows have their injected entries zeroed
    "large": Workload("large", T=4096, K=8192, N=28672, sigma=0.015, n_out=25, lo=20.0,
                      hi=80.0, threshold=6.0, seed=4, zero_rows=_cfg4_zero_rows(4096)),
    # outlier-fraction sweep; n_out in {0, 8, 64, 512}, threshold in {6, inf}
    "sweep": Workload("sweep", T=2048, K=14336, N=14336, sigma=0.01, n_out=8, lo=10.0,
                      hi=60.0, threshold=6.0, seed=5),
}

SWEEP_N_OUT = (0, 8, 64, 512)
SWEEP_THRESHOLDS = (6.0, math.inf)


def make_weight(rng: np.random.Generator, N: int, K: int, sigma: float) -> np.ndarray:
    """Step 1 of the recipe: fp16 weight matrix [N, K]."""
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w.astype(np.float16)


def make_activations(rng: np.random.Generator, T: int, K: int, n_out: int, lo: float,
                     hi: float, zero_rows: int = 0):
    """Steps 2-4 of the recipe: fp16 activations [T, K] and the injected columns."""
    cols = np.sort(rng.choice(K, size=n_out, replace=False)).astype(np.int64) if n_out else \
        np.zeros(0, np.int64)
    z = rng.standard_normal((T, K), dtype=np.float32)
    x = z.astype(np.float16)
    if n_out:
        mag = rng.uniform(lo, hi, size=(T, n_out)).astype(np.float32)
        sgn = np.where(z[:, cols] < 0, np.float32(-1), np.float32(1))
        x[:, cols] = (sgn * mag).astype(np.float16)
    rows = np.zeros(0, np.int64)
    if zero_rows and n_out:
        rows = np.sort(rng.choice(T, size=zero_rows, replace=False)).astype(np.int64)
        x[rows[:, None], cols[None, :]] = 0
    return x, cols, rows


def make_output_grad(seed: int, T: int, N: int) -> np.ndarray:
    """Step 5 of the recipe: fp16 output gradient [T, N] for the input-gradient checks."""
    g = rng_for(seed, 2).standard_normal((T, N), dtype=np.float32)
    return g.astype(np.float16)


def make_state(seed: int, n: int) -> np.ndarray:
    """Step 6 of the recipe: an fp32 optimizer-state-like tensor of n elements."""
    s = rng_for(seed, 3).standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    s[::1000] *= np.float32(50.0)
    return s


def as_bf16_input(x16: np.ndarray) -> np.ndarray:
    """Step 7 of the recipe: bf16 bit patterns (uint16) of fp16 draws, by truncation."""
    bits = np.ascontiguousarray(np.asarray(x16, dtype=np.float16).astype(np.float32)).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


def make_bias(seed: int, N: int, bf16: bool = False) -> np.ndarray:
    """Step 8 of the recipe: a bias vector [N], fp16 values or bf16 bit patterns."""
    b = rng_for(seed, 4).standard_normal(N, dtype=np.float32) * np.float32(0.5)
    if bf16:
        return (np.ascontiguousarray(b).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return b.astype(np.float16)


def rng_for(seed: int, stream: int) -> np.random.Generator:
    """Stream 0 draws the weight, 1 the activations, 2 output gradients, 3 codec
    states, 4 biases."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def make(w: Workload, T: int | None = None, with_weight: bool = True):
    """Draw (W, X) for a workload. ``T`` smaller than ``w.T`` keeps the first rows."""
    W = make_weight(rng_for(w.seed, 0), w.N, w.K, w.sigma) if with_weight else None
    X, cols, rows = make_activations(rng_for(w.seed, 1), w.T, w.K, w.n_out, w.lo, w.hi,
                                     w.zero_rows)
    if T is not None:
        X = np.ascontiguousarray(X[:T])
    return W, X, cols, rows


def random_fp16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """Plain normal fp16 array (for edge-shape tests)."""
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float16)


def random_fp16_large(rng: np.random.Generator, shape, scale: float = 1.0,
                      chunk: int = 1 << 26) -> np.ndarray:
    """Plain normal fp16 array drawn ``chunk`` elements at a time (inputs of several GB
    without a float32 copy of the whole)."""
    out = np.empty(shape, np.float16)
    flat = out.reshape(-1)
    for i in range(0, flat.size, chunk):
        n = min(chunk, flat.size - i)
        flat[i:i + n] = (rng.standard_normal(n, dtype=np.float32) * np.float32(scale)).astype(np.float16)
    return out
