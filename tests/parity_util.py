"""Parity bars for 16-bit outputs, shared by the GPU tests.

fp16 output: max-abs-relative error (oracle.parity_error) <= 1e-3.
bf16 output (8 significant bits): the kernel's fp32 sum and the oracle's exact
sum may straddle a rounding boundary, so every element must be the oracle's
bf16 value or one of its two neighbours (or within 2**-16 of the largest |Y|,
the fp32 arithmetic's own slack where terms cancel), at least 99% of the
elements must be bit-identical, and the max-abs-relative error must stay
<= 2**-7 (one bf16 step at the largest |Y|).
"""
from __future__ import annotations

import numpy as np

import oracle

F16_TOL = 1e-3
BF16_TOL = 2.0 ** -7
BF16_SLACK = 2.0 ** -16
BF16_EXACT_FRACTION = 0.99


def _ordered(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b >> 15 != 0, -mag, mag)


def check_y(Y, Y_ref, dtype):
    """Assert the bar above (fp16 values, or bf16 bit patterns as uint16); return the error."""
    if dtype == "f16":
        err = oracle.parity_error(Y, Y_ref)
        assert err <= F16_TOL, f"Y parity error {err}"
        return err
    got, want = oracle.bf16_bits_to_f32(Y), oracle.bf16_bits_to_f32(Y_ref)
    err = oracle.parity_error(got, want)
    assert err <= BF16_TOL, f"bf16 Y parity error {err}"
    if Y.size == 0:
        return err
    steps = np.abs(_ordered(Y) - _ordered(Y_ref))
    slack = BF16_SLACK * float(np.abs(want.astype(np.float64)).max())
    far = (steps > 1) & (np.abs(got.astype(np.float64) - want) > slack)
    assert not far.any(), f"{int(far.sum())} bf16 outputs more than one step away"
    same = float(np.mean(Y == Y_ref))
    assert same >= BF16_EXACT_FRACTION or int(np.sum(Y != Y_ref)) <= 1, \
        f"only {same:.4f} of bf16 outputs bit-identical"
    return err
