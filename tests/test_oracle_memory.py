"""Pins of the per-stage memory closed forms against the figures the pages print."""

import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
FIG = {f["id"]: f for f in GOLDEN["figures"]}
GIB = 1024 ** 3


def test_fp16_params_175b():
    f = FIG["fp16_params_175b"]
    est = O.estimate_memory_per_gpu(f["num_params"], 64)
    assert est["DP"].parameters * GIB == pytest.approx(f["bytes"], rel=1e-12)


def test_model_state_175b_is_16_bytes_per_param():
    f = FIG["model_state_175b"]
    est = O.estimate_memory_per_gpu(f["num_params"], 64)
    assert est["DP"].total * GIB == pytest.approx(f["bytes"], rel=f["rel_tol"])
    # the 2.1 TB of 12 bytes alone would miss the printed figure
    assert abs(est["DP"].optimizer_states * GIB - f["bytes"]) / f["bytes"] > 0.2


@pytest.mark.parametrize("fid,stage", [("zero1_saving", "ZeRO-1"), ("zero2_saving", "ZeRO-2")])
def test_saving_limits(fid, stage):
    lim = FIG[fid]["ratio_limit"]
    prev = 0.0
    for nd in (2, 8, 64, 1024, 1 << 20):
        est = O.estimate_memory_per_gpu(7e9, nd)
        r = est["DP"].total / est[stage].total
        assert prev < r < lim            # grows with Nd, never reaches the limit
        prev = r
    assert prev == pytest.approx(lim, rel=1e-4)


def test_zero3_linear_in_nd():
    for nd in (1, 3, 8, 64):
        est = O.estimate_memory_per_gpu(13e9, nd)
        assert est["ZeRO-3"].total == pytest.approx(est["DP"].total / nd, rel=1e-15)


def test_optimizer_state_is_12n_over_nd():
    f = FIG["opt_state_per_rank"]
    est = O.estimate_memory_per_gpu(7e9, 8)
    assert est["DP"].optimizer_states * GIB == pytest.approx(f["bytes_per_param"] * 7e9)
    for stage in ("ZeRO-1", "ZeRO-2", "ZeRO-3"):
        assert est[stage].optimizer_states == pytest.approx(est["DP"].optimizer_states / 8)


def test_stage1_ratio_7b_8_cards():
    f = FIG["llama7b_8cards_stage1"]
    p = O.partition_plan(7_000_000_000, f["dp_degree"])
    dp = O.stage_bytes_exact(p, 0)[0]
    z1 = O.stage_bytes_exact(p, 1)[0]
    assert z1 / dp == pytest.approx(f["after_gb"] / f["before_gb"], rel=1e-15)


def test_estimator_defaults_and_nd1_degenerate():
    f = FIG["estimator_defaults"]
    est = O.estimate_memory_per_gpu(1e9, 1)
    assert est["DP"].parameters * GIB == pytest.approx(f["bytes_per_param"] * 1e9)
    assert est["DP"].gradients * GIB == pytest.approx(f["bytes_per_param"] * 1e9)
    for stage in ("ZeRO-1", "ZeRO-2", "ZeRO-3"):   # one rank: nothing to shard
        assert est[stage] == est["DP"]


def test_components_per_stage():
    est = O.estimate_memory_per_gpu(1e9, 4)
    dp = est["DP"]
    assert est["ZeRO-1"].gradients == dp.gradients and est["ZeRO-1"].parameters == dp.parameters
    assert est["ZeRO-2"].gradients == pytest.approx(dp.gradients / 4)
    assert est["ZeRO-2"].parameters == dp.parameters
    assert est["ZeRO-3"].parameters == pytest.approx(dp.parameters / 4)


def test_exact_bytes_match_closed_form_without_padding():
    for model_n, nd in ((124_356_864, 8), (6_738_415_616, 8), (174_604_259_328, 64)):
        p = O.partition_plan(model_n, nd)
        assert p.pad == 0
        est = O.estimate_memory_per_gpu(model_n, nd)
        for stage, name in enumerate(("DP", "ZeRO-1", "ZeRO-2", "ZeRO-3")):
            opt, grad, par, tot = O.stage_bytes_exact(p, stage)
            assert tot == opt + grad + par
            assert tot / GIB == pytest.approx(est[name].total, rel=1e-14)


def test_exact_bytes_with_padding_use_shard_size():
    p = O.partition_plan(1_000_003, 4)
    assert O.stage_bytes_exact(p, 3) == (12 * 250_001, 2 * 250_001, 2 * 250_001, 16 * 250_001)
    assert O.stage_bytes_exact(p, 1, 2, 4, 12) == (12 * 250_001, 4 * 1_000_003, 2 * 1_000_003,
                                                   12 * 250_001 + 6 * 1_000_003)


def test_stage_choice_page_examples():
    f = FIG["stage_choice_examples"]
    usable = int(f["card_bytes"] * 0.75)
    for c in f["cases"]:
        plan = O.partition_plan(int(c["num_params"]), 8)
        stage, offload, b = O.choose_stage(plan, usable)
        assert (stage, offload) == (c["stage"], c["offload"]), c
        assert b == O.stage_bytes_exact(plan, stage)


def test_stage_choice_reserve_window_of_the_reading():
    """The reading's claim: at Nd = 8 every budget between the 13B ZeRO-2 footprint and the 13B
    ZeRO-1 footprint reproduces the page's three answers, and budgets outside it do not."""
    plans = {n: O.partition_plan(int(n), 8) for n in (7e9, 13e9, 70e9)}
    lo = O.stage_bytes_exact(plans[13e9], 2)[3]
    hi = O.stage_bytes_exact(plans[13e9], 1)[3]
    assert 0.10 < 1 - hi / 80e9 < 0.12 and 0.38 < 1 - lo / 80e9 < 0.40
    for usable in (lo, (lo + hi) // 2, hi - 1):
        got = [O.choose_stage(plans[n], usable)[:2] for n in (7e9, 13e9, 70e9)]
        assert got == [(1, False), (2, False), (3, True)]
    assert O.choose_stage(plans[13e9], hi)[0] == 1
    assert O.choose_stage(plans[13e9], lo - 1)[0] == 3


def test_stage_choice_is_monotone():
    """More parameters never pick a lower stage; a bigger budget never picks a higher one; more
    ranks never pick a higher one."""
    budgets = [int(x * 1e9) for x in (8, 16, 40, 60, 80, 160, 288)]
    sizes = [int(x * 1e9) for x in (0.1, 1, 7, 13, 34, 70, 175, 530)]
    for nd in (1, 2, 8, 64):
        for u in budgets:
            st = [O.choose_stage(O.partition_plan(n, nd), u) for n in sizes]
            keys = [(s, o) for s, o, _ in st]
            assert keys == sorted(keys)
        for n in sizes:
            st = [O.choose_stage(O.partition_plan(n, nd), u)[:2] for u in budgets]
            assert st == sorted(st, reverse=True)
    for n in sizes:
        for u in budgets:
            st = [O.choose_stage(O.partition_plan(n, nd), u)[:2] for nd in (1, 2, 4, 8, 16, 64)]
            assert st == sorted(st, reverse=True)


# ------------------------------------------------------------------ communication volume per step

def _ring_reduce_scatter(bufs):
    """Ring reduce-scatter, simulated: each rank's buffer is nd chunks; at step s rank r sends its
    chunk (r - s) mod nd to rank r + 1, which adds it to its own copy. Returns each rank's chunks
    afterwards and the elements each rank sent."""
    nd = len(bufs)
    chunks = [[c.copy() for c in b] for b in bufs]
    sent = [0] * nd
    for s in range(nd - 1):
        msgs = [(r, (r - s) % nd, chunks[r][(r - s) % nd].copy()) for r in range(nd)]
        for r, c, data in msgs:
            chunks[(r + 1) % nd][c] = chunks[(r + 1) % nd][c] + data
            sent[r] += data.size
    return chunks, sent


def _ring_all_gather(owned):
    """Ring all-gather, simulated: rank r starts with chunk (r + 1) mod nd (where a ring
    reduce-scatter leaves the reduced chunk) and at step s forwards chunk (r + 1 - s) mod nd."""
    nd = len(owned)
    have = [{(r + 1) % nd: owned[r].copy()} for r in range(nd)]
    sent = [0] * nd
    for s in range(nd - 1):
        msgs = [(r, (r + 1 - s) % nd, have[r][(r + 1 - s) % nd]) for r in range(nd)]
        for r, c, data in msgs:
            have[(r + 1) % nd][c] = data.copy()
            sent[r] += data.size
    return have, sent


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8, 9])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_ring_collectives_send_nd_minus_1_shards(nd, S):
    """Brute force: a simulated ring reduce-scatter leaves every rank one distinct, fully reduced
    chunk, a simulated all-gather then gives every rank every chunk, and each sends (nd - 1) * S
    elements per rank: the unit the closed form counts in."""
    rng = np.random.default_rng(nd * 100 + S)
    bufs = [[rng.integers(-50, 50, S) for _ in range(nd)] for _ in range(nd)]
    total = [sum(bufs[r][c] for r in range(nd)) for c in range(nd)]
    chunks, sent = _ring_reduce_scatter(bufs)
    owned = [chunks[r][(r + 1) % nd] for r in range(nd)]
    for r in range(nd):
        assert np.array_equal(owned[r], total[(r + 1) % nd])
    assert sent == [(nd - 1) * S] * nd
    have, sent_ag = _ring_all_gather(owned)
    for r in range(nd):
        assert sorted(have[r]) == list(range(nd))
        for c in range(nd):
            assert np.array_equal(have[r][c], total[c])
    assert sent_ag == [(nd - 1) * S] * nd
    # per stage, in units of one ring pass: DP all-reduce = reduce-scatter + all-gather
    plan = O.partition_plan(nd * S, nd)
    one = sent[0]
    for stage, (gp, pp) in enumerate(((2, 0), (1, 1), (1, 1), (1, 2))):
        assert O.stage_comm_bytes(plan, stage, param_b=2, grad_b=4) == (gp * one * 4, pp * one * 2,
                                                                        gp * one * 4 + pp * one * 2)


def check_comm_pins(comm=O.stage_comm_bytes):
    """The pins of the per-step communication closed form, for the oracle or a planted mutant.

    Unit: a simulated ring reduce-scatter (and all-gather) sends (nd - 1) * S elements per rank,
    and an all-reduce is one of each. Pages: ZeRO-1/2 send what DP sends, ZeRO-3 1.5 times that,
    a reduce-scatter half of an all-reduce, and ZeRO-1 all-gathers the updated parameters once
    after the optimizer step ([P1] section 二). One rank sends nothing.
    """
    for nd, S in ((2, 1), (3, 4), (5, 3)):
        rng = np.random.default_rng(nd)
        _, sent = _ring_reduce_scatter([[rng.integers(0, 9, S) for _ in range(nd)] for _ in range(nd)])
        plan = O.partition_plan(nd * S, nd)
        assert comm(plan, 0, 1, 1)[0] == 2 * sent[0]            # all-reduce = reduce-scatter + all-gather
        assert comm(plan, 1, 3, 1)[1] == 3 * sent[0]            # ZeRO-1: one all-gather of parameters
    r12, r3 = FIG["zero12_comm_equals_dp"]["ratio"], FIG["zero3_comm_ratio"]["ratio"]
    half = FIG["reduce_scatter_half_of_all_reduce"]["ratio"]
    for n, nd in ((1_000_003, 4), (124_356_864, 8), (6_738_415_616, 8), (174_604_259_328, 64), (7, 16)):
        plan = O.partition_plan(n, nd)
        dp = comm(plan, 0, 2, 2)
        z = [comm(plan, k, 2, 2) for k in (1, 2, 3)]
        assert z[0][2] == r12 * dp[2] and z[1][2] == r12 * dp[2]
        assert z[2][2] == r3 * dp[2]
        assert z[1][0] == half * dp[0]          # the gradient reduce-scatter is half the all-reduce
    for stage in range(4):
        assert comm(O.partition_plan(12345, 1), stage, 2, 2) == (0, 0, 0)


def test_comm_pins_hold_for_the_oracle():
    check_comm_pins()


def _comm_mutant(kind):
    def comm(plan, stage, param_b=2, grad_b=2):
        unit = plan.nd * plan.shard_elems if kind == "unit_nd" else (plan.nd - 1) * plan.shard_elems
        passes = {"zero3_one_gather": ((2, 0), (1, 1), (1, 1), (1, 1)),
                  "dp_reduce_scatter_only": ((1, 0), (1, 1), (1, 1), (1, 2)),
                  "zero1_all_reduce": ((2, 0), (2, 0), (1, 1), (1, 2))}.get(
            kind, ((2, 0), (1, 1), (1, 1), (1, 2)))
        gp, pp = passes[stage]
        g, w = gp * unit * grad_b, pp * unit * param_b
        return g, w, g + w
    return comm


@pytest.mark.parametrize("kind", ["unit_nd", "zero3_one_gather", "dp_reduce_scatter_only",
                                  "zero1_all_reduce"])
def test_comm_mutants_are_caught(kind):
    with pytest.raises(AssertionError):
        check_comm_pins(_comm_mutant(kind))


def test_comm_about_2n_per_step():
    """ZeRO-1/2 send about 2N elements per rank per step: 2 (nd - 1) / nd of N, rising to 2."""
    lim = FIG["zero12_comm_2n"]["elements_per_param"]
    prev = 0.0
    n = 2 ** 40
    for nd in (2, 8, 64, 1024, 1 << 16):
        plan = O.partition_plan(n, nd)
        r = O.stage_comm_bytes(plan, 1, param_b=1, grad_b=1)[2] / n
        assert r == 2 * (nd - 1) / nd and prev < r < lim
        prev = r
    assert prev == pytest.approx(lim, rel=1e-4)


def test_comm_single_rank_sends_nothing():
    plan = O.partition_plan(12345, 1)
    for stage in range(4):
        assert O.stage_comm_bytes(plan, stage) == (0, 0, 0)
    with pytest.raises(ValueError):
        O.stage_comm_bytes(plan, 4)
