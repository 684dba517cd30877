"""Bit-pattern comparisons for the parity tests (no torch, usable on the CPU)."""

import numpy as np


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"{what}: {bad.size} of {want.size} differ; first at {bad[:5].tolist()}: "
                             f"got {[hex(int(x)) for x in got[bad[:5]]]} want {[hex(int(x)) for x in want[bad[:5]]]}")


_NAN_ABOVE = {32: (0x7FFFFFFF, 0x7F800000), "bf16": (0x7FFF, 0x7F80), "f16": (0x7FFF, 0x7C00)}


def is_nan_bits(bits: np.ndarray, kind) -> np.ndarray:
    """NaN test on raw bit patterns: kind 32 (fp32), "bf16" or "f16"."""
    mask, inf = _NAN_ABOVE[kind]
    return (bits.astype(np.uint32) & mask) > inf


def assert_bits_equal_nan(got: np.ndarray, want: np.ndarray, what: str, kind=32):
    """Bit equality, except that where the expected value is a NaN any NaN is accepted: the host's
    and the GPU's default NaN differ in sign, and NaN payloads carry no value."""
    wn, gn = is_nan_bits(want, kind), is_nan_bits(got, kind)
    if not np.array_equal(wn, gn):
        bad = np.nonzero(wn != gn)[0]
        raise AssertionError(f"{what}: NaN positions differ at {bad.size} elements, first {bad[:5].tolist()}: "
                             f"got {[hex(int(x)) for x in got[bad[:5]]]} want {[hex(int(x)) for x in want[bad[:5]]]}")
    keep = ~wn
    assert_bits_equal(got[keep], want[keep], what)
