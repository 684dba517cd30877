"""Plant plausible mistakes in copies of the oracle and check that the pins catch every one.

Nothing here changes the oracle itself: each mutant is a local, deliberately wrong function run
through the same checks the oracle passes (tests/adam_pins.py and the cast/sum pins).
"""

import dataclasses
import math

import numpy as np
import pytest

import oracle as O
import adam_pins as P
import clip_pins as CP


def _scalars_with(**over):
    def fn(hp):
        s = O.adam_scalars(hp)
        vals = {k: (v(hp) if callable(v) else v) for k, v in over.items()}
        return dataclasses.replace(s, **{k: np.float32(v) for k, v in vals.items()})
    return fn


def _update_variant(kind):
    def upd(p, m, v, g, sc, wd_mode="adamw"):
        if wd_mode == "l2":
            g = g - sc.w * p if kind == "l2_sign" else g + sc.w * p
        if kind == "swap_betas":
            m = sc.b2 * m + sc.c2 * g
            v = sc.b1 * v + sc.c1 * (g * g)
        elif kind == "transposed_m":
            m = sc.c1 * m + sc.b1 * g
            v = sc.b2 * v + sc.c2 * (g * g)
        elif kind == "v_not_squared":
            m = sc.b1 * m + sc.c1 * g
            v = sc.b2 * v + sc.c2 * np.abs(g)
        else:
            m = sc.b1 * m + sc.c1 * g
            v = sc.b2 * v + sc.c2 * (g * g)
        if kind == "eps_in_sqrt":
            den = np.sqrt(v / (sc.bc * sc.bc) + sc.e)
        elif kind == "eps_before_correction":
            den = (np.sqrt(v) + sc.e) / sc.bc
        else:
            den = np.sqrt(v) / sc.bc + sc.e
        if wd_mode == "adamw" and kind != "decay_after":
            p = p * sc.dec
        upd_ = sc.ss * (m / den)
        p = p + upd_ if kind == "sign" else p - upd_
        if wd_mode == "adamw" and kind == "decay_after":
            p = p * sc.dec
        return p, m, v
    return upd


MUTANTS = {
    "no_bias_correction_1": (O.adam_update, _scalars_with(ss=lambda hp: hp.lr)),
    "no_bias_correction_2": (O.adam_update, _scalars_with(bc=1.0)),
    "step_from_zero": (O.adam_update, _scalars_with(
        ss=lambda hp: hp.lr / (1 - hp.beta1 ** (hp.step + 1)),
        bc=lambda hp: math.sqrt(1 - hp.beta2 ** (hp.step + 1)))),
    "decay_uses_wd_only": (O.adam_update, _scalars_with(dec=lambda hp: 1 - hp.weight_decay)),
    "swap_betas": (_update_variant("swap_betas"), O.adam_scalars),
    "transposed_m": (_update_variant("transposed_m"), O.adam_scalars),
    "v_not_squared": (_update_variant("v_not_squared"), O.adam_scalars),
    "eps_in_sqrt": (_update_variant("eps_in_sqrt"), O.adam_scalars),
    "eps_before_correction": (_update_variant("eps_before_correction"), O.adam_scalars),
    "sign": (_update_variant("sign"), O.adam_scalars),
    "decay_after": (_update_variant("decay_after"), O.adam_scalars),
    "l2_sign": (_update_variant("l2_sign"), O.adam_scalars),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_adam_mutant_is_caught(name):
    upd, scal = MUTANTS[name]
    caught = []
    with np.errstate(all="ignore"):
        for check_name, check in P.ALL_CHECKS.items():
            try:
                check(upd, scal)
            except AssertionError:
                caught.append(check_name)
    assert caught, f"mutant {name} passed every pin"


def test_cast_mutants_are_caught():
    x = np.float32([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9, (2 - 2.0 ** -8) * 2.0 ** 127])
    want = O.cast_bf16_rne(x)
    truncate = (x.view(np.uint32) >> 16).astype(np.uint16)
    ties_away = ((x.view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    assert not np.array_equal(truncate, want)
    assert not np.array_equal(ties_away, want)
    # the expected patterns come from the brute-force nearest-even search of the cast pins
    assert want.tolist() == [0x3F80, 0x3F82, 0x3F80, 0x7F80]


def test_sum_mutants_are_caught():
    a = [np.float32([1.0]), np.float32([2.0 ** 24]), np.float32([-(2.0 ** 24)])]
    rev = a[-1] + a[-2] + a[0]
    mean = O.replica_sum(a, "f32") / np.float32(3)
    assert rev[0] != O.replica_sum(a, "f32")[0] or mean[0] != 0.0
    k = np.arange(-8, 8, dtype=np.float32).reshape(4, 4) * np.float32(0.25)
    assert not np.array_equal(O.replica_sum(list(k), "f32") / np.float32(4), k.sum(0))


def _clip_variant(kind):
    """Plausible mistakes in the clip rule min(1, max_norm / (sqrt(sq) + eps))."""
    def clip(total_sq, max_norm=1.0, eps=1e-6):
        if kind == "eps_inside_sqrt":
            q = max_norm / math.sqrt(total_sq + eps)
        elif kind == "eps_dropped":
            q = max_norm / math.sqrt(total_sq) if total_sq > 0 else math.inf
        elif kind == "squared_norm_as_norm":
            q = max_norm / (total_sq + eps)
        else:
            q = max_norm / (math.sqrt(total_sq) + eps)
        return max(1.0, q) if kind == "max_for_min" else min(1.0, q)
    return clip


@pytest.mark.parametrize("kind", ["eps_inside_sqrt", "eps_dropped", "squared_norm_as_norm", "max_for_min"])
def test_clip_mutant_is_caught(kind):
    caught = []
    for check_name, check in CP.ALL_CHECKS.items():
        try:
            check(_clip_variant(kind))
        except AssertionError:
            caught.append(check_name)
    assert caught, f"clip mutant {kind} passed every pin"


def test_clip_unmutated_variant_passes():
    """The mutants' own scaffold, unmutated, passes every pin (so a caught mutant is caught for its
    mistake, not for the scaffold)."""
    for check in CP.ALL_CHECKS.values():
        check(_clip_variant("none"))
