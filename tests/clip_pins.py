"""Checks that pin the oracle's clip coefficient to a library routine outside it.

No page defines gradient clipping; the reading is the global-norm rule with eps added to the norm
and the coefficient capped at 1. torch.nn.utils.clip_grad_norm_ implements that rule
independently: it forms the total L2 norm of the gradients itself, divides max_norm by
(norm + 1e-6) and clamps the result at 1, then scales every gradient by it.

Each check takes the clip function as an argument (defaulting to the oracle's), so the mutation
tests can run the same checks against deliberately wrong copies and see them fail.

Two kinds of case:
  * exact: a gradient (3*2^k, 4*2^k) has norm 5*2^k exactly and squared norm 25*4^k exactly, so
    both sides start from the same fp64 denominator d = 5*2^k + 1e-6; the coefficient torch applied
    is read back exactly from the power-of-two element (4*2^k times the coefficient is an exact
    product). torch forms max_norm / d as max_norm * (1/d), two roundings, so it is held to 2 ulps;
    the oracle's quotient must also be the correctly rounded max_norm / d, found with exact
    rational arithmetic.
  * random: gradients of a few thousand N(0, s) elements over several tensors, where the two sides
    sum the squares in different orders; the coefficients agree to a few fp64 ulps.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import oracle as O

EPS = 1e-6    # torch's clip_grad_norm_ adds this to the norm
# powers of two for the exact cases: tiny, ordinary and huge norms
EXACT_K = (-60, -40, -30, -20, -12, -3, 0, 2, 10, 40, 60)
MAX_NORMS = (1e-7, 1e-3, 0.5, 1.0, 5.0, 1e4)


def _torch_coef(grads: list[np.ndarray], max_norm: float, probe: tuple[int, int] | None = None):
    """(coefficient torch applied, its total norm) for fp64 CPU gradients.

    probe = (tensor, element) of a power-of-two gradient entry: the coefficient is then read back
    exactly as scaled / original. Without it, the ratio on the largest entry is returned."""
    params = []
    for g in grads:
        p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
        p.grad = torch.from_numpy(g.astype(np.float64).copy())
        params.append(p)
    norm = float(torch.nn.utils.clip_grad_norm_(params, max_norm, norm_type=2.0))
    if probe is None:
        t = max(range(len(grads)), key=lambda i: np.abs(grads[i]).max())
        probe = (t, int(np.argmax(np.abs(grads[t]))))
    t, i = probe
    return float(params[t].grad[i]) / float(grads[t][i]), norm


def check_exact_norms(clip_fn=O.clip_coefficient):
    """Norms 5*2^k (exact) below, at and above each max_norm: torch's coefficient to 2 ulps, and
    the correctly rounded quotient of the same fp64 operands exactly."""
    checked = 0
    for k in EXACT_K:
        s = 2.0 ** k
        g = np.array([3.0 * s, 4.0 * s])
        sq = 25.0 * s * s                          # exact: 25 needs 5 bits
        d = 5.0 * s + EPS                          # one fp64 rounding, the same on both sides
        for max_norm in MAX_NORMS + (5.0 * s,):    # the last: the norm equals max_norm
            want, norm = _torch_coef([g], max_norm, probe=(0, 1))
            assert norm == 5.0 * s, (k, norm)
            got = clip_fn(sq, max_norm=max_norm, eps=EPS)
            assert abs(got - want) <= 2 * math.ulp(want), \
                f"k={k} max_norm={max_norm}: got {got!r}, torch applied {want!r}"
            exact = min(1.0, float(Fraction(max_norm) / Fraction(d)))   # float() rounds to nearest
            assert got == exact, f"k={k} max_norm={max_norm}: got {got!r}, correctly rounded {exact!r}"
            checked += 1
    assert checked == len(EXACT_K) * (len(MAX_NORMS) + 1)


def check_split_tensors(clip_fn=O.clip_coefficient):
    """The norm over several tensors is the norm of their concatenation (torch takes the norm of
    the per-tensor norms): 3*2^k and 4*2^k in separate tensors give the same coefficient."""
    for k in (-20, 0, 7):
        s = 2.0 ** k
        for max_norm in (1e-3, 1.0, 100.0):
            want, norm = _torch_coef([np.array([3.0 * s]), np.array([4.0 * s])], max_norm, probe=(1, 0))
            assert norm == 5.0 * s
            assert abs(clip_fn(25.0 * s * s, max_norm=max_norm, eps=EPS) - want) <= 2 * math.ulp(want)


def check_random_grads(clip_fn=O.clip_coefficient, seed=11):
    """Random gradients over three tensors, norms from 1e-9 to 1e6 against max_norm 1: equal to
    a few fp64 ulps (the two sides sum the squares in different orders)."""
    rng = np.random.default_rng(seed)
    for scale in (1e-11, 1e-8, 1e-5, 1e-3, 1e-2, 0.1, 1.0, 1e4):
        grads = [rng.standard_normal(n) * scale for n in (1000, 37, 4096)]
        sq = math.fsum(float(x) * float(x) for g in grads for x in g)
        want, norm = _torch_coef(grads, 1.0)
        assert abs(math.sqrt(sq) - norm) <= 1e-15 * norm
        got = clip_fn(sq, max_norm=1.0, eps=EPS)
        # the norms' summation orders, torch's reciprocal and the probe ratio each add roundings
        assert abs(got - want) <= 4e-15 * want, f"scale {scale}: got {got!r}, torch {want!r}"


def check_limits(clip_fn=O.clip_coefficient):
    """Below max_norm the coefficient is exactly 1, as torch's clamp gives."""
    for sq in (0.0, 1e-30, 0.25, 0.999 ** 2):
        assert clip_fn(sq, max_norm=1.0, eps=EPS) == 1.0
    want, _ = _torch_coef([np.array([0.75 * 0.5, 0.5])], 1.0, probe=(0, 1))
    assert want == 1.0


ALL_CHECKS = {
    "exact_norms": check_exact_norms,
    "split_tensors": check_split_tensors,
    "random_grads": check_random_grads,
    "limits": check_limits,
}
