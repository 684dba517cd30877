"""The synthetic workloads have the sizes their model labels state."""

import numpy as np

import oracle as O
from workloads import WORKLOADS, flat_count, init_ranges, param_list
from workloads import host as H


def test_model_counts_match_labels():
    assert flat_count("gpt2-small") == 124_356_864            # "124M"
    assert flat_count("llama-7b") == 6_738_415_616            # "6.74B"
    assert flat_count("llama-13b") == 13_015_864_320          # "13B"
    assert flat_count("gpt3-175b") == 174_604_259_328         # "175B"


def test_shard_sizes():
    want = {"tiny": 250_001, "gpt2": 15_544_608, "llama7b": 842_301_952,
            "llama13b": 813_491_520, "gpt3": 2_728_191_552}
    for name, w in WORKLOADS.items():
        assert O.partition_plan(w.n, w.nd).shard_elems == want[name]
    g3 = WORKLOADS["gpt3"]
    s = O.partition_plan(g3.n, g3.nd).shard_elems
    assert s // g3.window == 40 and s % g3.window == 43_836_992


def test_init_ranges_cover_norms_and_biases():
    n_one = sum(n for _, n, k in param_list("llama-7b") if k == "one")
    assert n_one == 65 * 4096
    assert sum(e - s for s, e, k in init_ranges("llama-7b") if k == "one") == n_one
    assert sum(e - s for s, e, k in init_ranges("gpt2-small") if k == "zero") == 25 * 768


def test_host_generator_is_seeded_and_pads_with_zero():
    w = WORKLOADS["tiny"]
    a = H.flat_inputs(w, 1_000_004)
    b = H.flat_inputs(w, 1_000_004)
    assert np.array_equal(a["master"], b["master"]) and np.array_equal(a["grad"], b["grad"])
    assert a["master"][-1] == 0 and a["grad"][-1] == 0
    r = H.rank_inputs(WORKLOADS["gpt2"], 3 * 15_544_608, 4096, 4096)
    assert r["reps"].shape == (8, 4096) and r["reps"].dtype == np.uint16
