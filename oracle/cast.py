"""fp32 -> 16-bit casts of the updated parameters.  TEST INFRASTRUCTURE.

The pages keep 16-bit parameters beside an fp32 master copy ([P1] "ZeRO 优化器的三个阶段深度对比",
sections 一 and 二: 2 bytes per parameter next to the fp32 copy, m and v; [P3] "ZeRO Optimization",
comparisons: mixed precision combines with ZeRO). They say nothing about rounding.

Reading: IEEE round-to-nearest, ties to even, for both formats.
  bf16: keep the top 16 bits of the fp32 pattern after adding 0x7FFF plus the lowest kept bit
        (carry into the exponent gives the correct overflow to infinity); a NaN keeps its sign and
        top payload bits and gets the quiet bit 0x0040.
  fp16: IEEE binary16 with gradual underflow; magnitudes at or above 65520 become infinity.

Both are returned as uint16 bit patterns. Pinned in the CPU tests against a brute-force search for
the nearest representable value over the whole 16-bit code space (ties to even), against torch's
CPU conversions, and against hand-listed special values.
"""

from __future__ import annotations

import numpy as np


def cast_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # No uint32 wrap: the largest non-NaN pattern is 0xFF800000, far below 2**32 - 0x8000.
    rounded = (np.where(is_nan, np.uint32(0), u) + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    quiet = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def cast_fp16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 array -> IEEE binary16 bit patterns (uint16), round to nearest even."""
    with np.errstate(over="ignore"):                # overflow to infinity is the defined result
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact: the pattern is the top half of an fp32 pattern)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen_fp16(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> fp32 (exact)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
