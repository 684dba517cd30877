"""Pins of the ZeRO-3 gather oracle: a per-element brute force of the shard layout, the union of
all shards, and the layer ranges of the model shapes."""

import numpy as np
import pytest

import oracle as O
from workloads import layer_ranges, flat_count, MODELS


def _brute(shards, begin, count):
    S = len(shards[0])
    return np.array([shards[j // S][j % S] for j in range(begin, begin + count)], dtype=shards[0].dtype)


@pytest.mark.parametrize("nd,S", [(1, 7), (3, 5), (8, 16), (5, 1)])
def test_gather_matches_brute_force(nd, S):
    rng = np.random.default_rng(nd * 100 + S)
    shards = [rng.integers(0, 1 << 16, S, dtype=np.uint16) for _ in range(nd)]
    P = nd * S
    for begin in range(P + 1):
        for count in range(P - begin + 1):
            got = O.gather_range(shards, begin, count)
            assert np.array_equal(got, _brute(shards, begin, count)), (begin, count)


def test_gather_of_everything_is_the_partition_union():
    n, nd = 1003, 4
    plan = O.partition_plan(n, nd)
    flat = np.arange(plan.padded_n, dtype=np.float32)
    shards = []
    for r in range(nd):
        b, _ = O.shard_range(plan, r)
        shards.append(flat[b:b + plan.shard_elems])
    assert np.array_equal(O.gather_range(shards, 0, plan.padded_n), flat)
    assert np.array_equal(O.gather_range(shards, 0, n), flat[:n])


def test_gather_rejects_bad_ranges():
    shards = [np.zeros(4, np.uint16)] * 2
    for b, c in ((-1, 1), (0, 9), (8, 1)):
        with pytest.raises(ValueError):
            O.gather_range(shards, b, c)
    with pytest.raises(ValueError):
        O.gather_range([np.zeros(4), np.zeros(3)], 0, 1)


@pytest.mark.parametrize("model", sorted(MODELS))
def test_layer_ranges_tile_the_flat_space(model):
    r = layer_ranges(model)
    assert r[0][1] == 0 and r[-1][2] == flat_count(model)
    assert all(a[2] == b[1] for a, b in zip(r, r[1:]))
    assert all(e > s for _, s, e in r)
