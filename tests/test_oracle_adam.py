"""Pins of the oracle's replica sum, squared norm, overflow flag, Adam update and whole step."""

import math

import numpy as np
import pytest

import oracle as O
import clip_pins as CP
import adam_pins as P
from workloads import WORKLOADS
from workloads import host as H


@pytest.mark.parametrize("name", sorted(P.ALL_CHECKS))
def test_adam_pins(name):
    P.ALL_CHECKS[name](O.adam_update, O.adam_scalars)


def test_scalars_rounded_once_from_fp64():
    hp = O.AdamHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=11)
    s = O.adam_scalars(hp)
    assert s.ss == np.float32(3e-4 / (1 - 0.9 ** 11))
    assert s.bc == np.float32(math.sqrt(1 - 0.95 ** 11))
    assert s.dec == np.float32(1 - 3e-4 * 0.1) and s.c2 == np.float32(0.05)
    with pytest.raises(ValueError):
        O.adam_scalars(O.AdamHParams(step=0))


def test_replica_sum_identity_and_order():
    x = np.float32([1.5, -2.0, 3.25])
    assert np.array_equal(O.replica_sum([x], "f32"), x)
    # left-to-right order is visible: (1 + 2^24) rounds to 2^24 (ties to even), minus 2^24 is 0;
    # any other order would give 1
    a = [np.float32([1.0]), np.float32([2.0 ** 24]), np.float32([-(2.0 ** 24)])]
    assert O.replica_sum(a, "f32")[0] == 0.0
    assert O.replica_sum(a[::-1], "f32")[0] == 1.0


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_replica_sum_exact_on_dyadic_values(dtype):
    # values k * 2^-10 with |k| < 128 are exact in every format and their sums stay exact in fp32
    rng = np.random.default_rng(5)
    k = rng.integers(-127, 128, size=(16, 5000))
    vals = k.astype(np.float32) * np.float32(2.0 ** -10)
    if dtype == "f32":
        reps = list(vals)
    elif dtype == "bf16":
        reps = [(r.view(np.uint32) >> 16).astype(np.uint16) for r in vals]
    else:
        reps = [r.astype(np.float16).view(np.uint16) for r in vals]
    got = O.replica_sum(reps, dtype)
    assert np.array_equal(got.astype(np.float64), k.sum(0) * 2.0 ** -10)


def test_replica_sum_error_bound():
    rng = np.random.default_rng(6)
    reps = [(rng.standard_normal(20000) * 1e-3).astype(np.float32) for _ in range(64)]
    got = O.replica_sum(reps, "f32").astype(np.float64)
    exact = np.sum(np.stack(reps).astype(np.float64), axis=0)
    bound = 63 * 2.0 ** -24 * np.sum(np.abs(np.stack(reps)).astype(np.float64), axis=0)
    assert (np.abs(got - exact) <= bound).all()


def test_nonfinite_flag():
    base = np.zeros(100, np.float32)
    assert not O.nonfinite_flag(base)
    for bad in (np.inf, -np.inf, np.nan):
        x = base.copy()
        x[37] = bad
        assert O.nonfinite_flag(x)
    # +inf in one replica and -inf in another sum to NaN, still flagged
    a, b = base.copy(), base.copy()
    a[3], b[3] = np.inf, -np.inf
    s = O.replica_sum([a, b], "f32")
    assert np.isnan(s[3]) and O.nonfinite_flag(s)


def test_sqnorm_against_exact_sum():
    rng = np.random.default_rng(7)
    for n in (0, 1, 7, 1000, 300_001):
        a = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        for s in (1.0, 2.0 ** -16, 0.3):
            terms = [(float(x) * s) ** 2 for x in a.tolist()]
            want = math.fsum(terms)
            got = O.shard_sqnorm(a, s)
            assert got == pytest.approx(want, rel=1e-14, abs=0)


def test_sqnorm_closed_forms():
    a = np.full(12345, 0.75, np.float32)
    assert O.shard_sqnorm(a) == 12345 * 0.5625
    assert O.shard_sqnorm(np.concatenate([a, np.zeros(99, np.float32)])) == 12345 * 0.5625
    assert O.shard_sqnorm(a, 2.0 ** -16) == 12345 * 0.5625 * 2.0 ** -32


def test_clip_coefficient_ieee_edges():
    # IEEE edges: a zero norm with eps = 0 is not clipped, an infinite norm scales to 0, NaN gives 1
    assert O.clip_coefficient(0.0, max_norm=1.0, eps=0.0) == 1.0
    assert O.clip_coefficient(float("inf")) == 0.0
    assert O.clip_coefficient(float("nan")) == 1.0
    # with eps = 0 and a perfect-square norm the quotient is exact
    assert O.clip_coefficient(16.0, max_norm=1.0, eps=0.0) == 0.25
    assert O.clip_coefficient(2.0 ** -40, max_norm=2.0 ** -30, eps=0.0) == 2.0 ** -10


@pytest.mark.parametrize("check", sorted(CP.ALL_CHECKS))
def test_clip_coefficient_against_torch(check):
    """The clip rule against torch.nn.utils.clip_grad_norm_ (fp64 CPU gradients): exact norms
    below, at and above max_norm, tiny and huge norms, several tensors, random gradients."""
    CP.ALL_CHECKS[check]()


def test_union_of_shards_equals_unsharded_tiny():
    """ZeRO changes where state lives, not the arithmetic: the 4 rank shards of the tiny workload,
    stepped 3 times each, concatenate to the unsharded update, bit for bit, padding left inert."""
    w = WORKLOADS["tiny"]
    plan = O.partition_plan(w.n, w.nd)
    flat = H.flat_inputs(w, plan.padded_n)
    S = plan.shard_elems
    for out_dtype in w.out_dtypes:
        p_full, m_full, v_full = flat["master"], np.zeros(plan.padded_n, np.float32), np.zeros(plan.padded_n, np.float32)
        shards = [(flat["master"][r * S:(r + 1) * S].copy(), np.zeros(S, np.float32), np.zeros(S, np.float32))
                  for r in range(w.nd)]
        for t in range(1, w.steps + 1):
            hp = O.AdamHParams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                               weight_decay=w.weight_decay, step=t)
            p_full, m_full, v_full, out_full = O.unsharded_step(flat["grad"], p_full, m_full, v_full, hp,
                                                                 out_dtype=out_dtype)
            gathered = np.empty(plan.padded_n, np.uint16)
            for r in range(w.nd):
                b, _ = O.shard_range(plan, r)
                p, m, v, out = O.sharded_step([flat["grad"][b:b + S]], "f32", 1.0, *shards[r], hp, out_dtype)
                shards[r] = (p, m, v)
                gathered[b:b + S] = out
            assert np.array_equal(np.concatenate([s[0] for s in shards]), p_full)
            assert np.array_equal(np.concatenate([s[1] for s in shards]), m_full)
            assert np.array_equal(np.concatenate([s[2] for s in shards]), v_full)
            assert np.array_equal(gathered, out_full)
            assert p_full[w.n:].tolist() == [0.0] * plan.pad and gathered[w.n:].tolist() == [0] * plan.pad


def test_skip_leaves_state_unchanged():
    rng = np.random.default_rng(8)
    p = rng.standard_normal(100).astype(np.float32)
    m = rng.standard_normal(100).astype(np.float32)
    v = np.abs(rng.standard_normal(100)).astype(np.float32)
    rep = np.full(100, np.inf, np.float32)
    p2, m2, v2, out = O.sharded_step([rep], "f32", 1.0, p, m, v, O.AdamHParams(), "bf16", skip=True)
    assert np.array_equal(p2, p) and np.array_equal(m2, m) and np.array_equal(v2, v) and out is None
