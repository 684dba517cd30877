"""Pins of the per-stage memory closed forms against the figures the pages print."""

import json
import os

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
