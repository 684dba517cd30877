"""Pins of the oracle's partition (even contiguous split, tail padding) by brute force."""

import itertools

import numpy as np
import pytest

import oracle as O

ALIGNS = (1, 2, 4, 8, 64, 256)


def _smallest_shard(n, nd, align):
    # brute force: the smallest multiple of align that gives every rank an equal share covering n
    s = 0
    while s * nd < n:
        s += align
    return s


@pytest.mark.parametrize("align", ALIGNS)
def test_partition_brute_force(align):
    for n in list(range(0, 64)) + list(range(64, 301, 7)):
        for nd in range(1, 18):
            p = O.partition_plan(n, nd, align)
            assert p.shard_elems == _smallest_shard(n, nd, align)
            assert p.shard_elems % align == 0
            assert p.padded_n == p.shard_elems * nd
            assert p.pad == p.padded_n - n and 0 <= p.pad < nd * align
            owner = np.full(p.padded_n, -1)
            real = 0
            for r in range(nd):
                b, valid = O.shard_range(p, r)
                assert b == r * p.shard_elems
                assert (owner[b:b + p.shard_elems] == -1).all()   # disjoint
                owner[b:b + p.shard_elems] = r
                # the real elements of a rank are its leading ones, and they tile [0, n) in order
                assert valid == max(0, min(p.shard_elems, n - b))
                real += valid
            assert (owner >= 0).all()                              # union is [0, P)
            assert real == n


def test_tiny_workload_values():
    p = O.partition_plan(1_000_003, 4)
    assert (p.shard_elems, p.padded_n, p.pad) == (250_001, 1_000_004, 1)
    assert O.shard_range(p, 3) == (750_003, 250_000)
    p8 = O.partition_plan(1_000_003, 4, 8)
    assert (p8.shard_elems, p8.padded_n, p8.pad) == (250_008, 1_000_032, 29)


def test_each_rank_holds_one_nd_th():
    # P1 section 二 / P3 definition: with no padding every rank holds exactly 1/Nd of the state
    for n, nd in itertools.product((8, 64, 6_738_415_616), (1, 2, 4, 8)):
        p = O.partition_plan(n, nd)
        assert p.pad == 0 and p.shard_elems * nd == n


def test_fewer_elements_than_ranks():
    p = O.partition_plan(3, 8)
    assert p.shard_elems == 1 and p.padded_n == 8 and p.pad == 5
    assert [O.shard_range(p, r)[1] for r in range(8)] == [1, 1, 1, 0, 0, 0, 0, 0]


def test_empty_space():
    p = O.partition_plan(0, 4)
    assert (p.shard_elems, p.padded_n, p.pad) == (0, 0, 0)


def test_invalid_and_overflow():
    with pytest.raises(ValueError):
        O.partition_plan(10, 0)
    with pytest.raises(ValueError):
        O.partition_plan(10, 2, 0)
    with pytest.raises(OverflowError):
        O.partition_plan((1 << 64) - 1, 3, 1 << 31)
    # the largest space that still fits: 2**64 - 2**10 over 2**10 ranks
    p = O.partition_plan((1 << 64) - 1024, 1024)
    assert p.padded_n == (1 << 64) - 1024
