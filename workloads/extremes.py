"""Seeded fp32 inputs spread over the whole binary32 range, for exercising the update's arithmetic
where IEEE special cases decide the result: subnormal operands and results, overflow to infinity,
0/0 and inf/inf, signed zeros.

Values are drawn as bit patterns: a random sign (or +), a biased exponent field uniform over a
chosen interval (0 means zero or subnormal, 254 the top binade) and a uniform 23-bit mantissa.
Input recipes only; nothing here computes any part of the step.
"""

from __future__ import annotations

import numpy as np

# (lo, hi) ranges of the biased exponent field per named regime
REGIMES = {
    "tiny": (0, 12),        # zeros, subnormals and the lowest normal binades
    "sq_sub": (50, 66),     # squares land in or next to the subnormal range
    "huge": (230, 254),     # up to FLT_MAX; products and squares overflow
    "full": (0, 254),       # every finite binade
    "mid": (100, 135),      # ordinary magnitudes, for the operands a regime leaves alone
}


# (regimes of g, p, m, v), grad scale, hyper-parameter overrides; each case aims at one special path
EXTREME_CASES = [
    (("tiny", "mid", "tiny", "tiny"), 1.0, dict(eps=0.0)),           # sqrt of subnormal v, tiny den
    (("sq_sub", "mid", "tiny", "tiny"), 1.0, dict(eps=0.0)),         # g*g subnormal or underflowing
    (("tiny", "tiny", "tiny", "tiny"), 1.0, dict(eps=1.0, weight_decay=0.0)),  # subnormal p and m out
    (("tiny", "mid", "tiny", "tiny"), 2.0 ** -16, dict(eps=0.0, wd_mode="l2", weight_decay=0.5)),
    (("mid", "mid", "mid", "mid"), 1e-42, dict(eps=0.0)),            # a subnormal grad scale
    (("huge", "mid", "huge", "huge"), 1.0, dict(eps=1e-8)),          # v overflows: the step vanishes
    (("huge", "huge", "mid", "mid"), 1.0, dict(eps=1e-8, wd_mode="l2", weight_decay=2.0)),  # inf/inf
    (("full", "full", "full", "full"), 1.0, dict(eps=1e-8, step=1)),
    (("full", "full", "full", "full"), 1.0, dict(eps=0.0, step=10 ** 6)),
    (("full", "full", "full", "full"), 2.0 ** -16, dict(eps=1e-8, lr=1.0, weight_decay=1.0)),  # dec = 0
]


def f32_patterns(rng: np.random.Generator, n: int, regime: str, nonneg: bool = False) -> np.ndarray:
    """n finite fp32 values with exponent fields uniform over REGIMES[regime]."""
    lo, hi = REGIMES[regime]
    exp = rng.integers(lo, hi + 1, n, dtype=np.uint32)
    mant = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    bits = (exp << 23) | mant
    if not nonneg:
        bits |= rng.integers(0, 2, n, dtype=np.uint32) << 31
    return bits.view(np.float32)


def mixed_state(rng: np.random.Generator, n: int, regimes: tuple[str, str, str, str]):
    """(g, p, m, v) with each array drawn from its own regime; v is non-negative."""
    g = f32_patterns(rng, n, regimes[0])
    p = f32_patterns(rng, n, regimes[1])
    m = f32_patterns(rng, n, regimes[2])
    v = f32_patterns(rng, n, regimes[3], nonneg=True)
    return g, p, m, v


def f16_all_patterns() -> np.ndarray:
    """Every binary16 bit pattern, infinities and NaNs included (uint16)."""
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
