"""Property-based checks (hypothesis) of the library's host entry points against the oracle, over
random sizes far beyond the fixed cases: the partition plan and shard ranges, per-stage bytes, the
stage choice, the fp32 Adam constants, and the arena layout's invariants. No GPU."""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
import zero_partition_plan_amd as Z

SETTINGS = settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
sizes = st.one_of(st.integers(0, 1 << 20), st.integers(0, 1 << 40), st.integers(0, (1 << 63) - 1))


@SETTINGS
@given(n=sizes, nd=st.integers(1, 1 << 16), align=st.integers(1, 1 << 12))
def test_plan_and_ranges_match_oracle(n, nd, align):
    try:
        want = O.partition_plan(n, nd, align)
    except OverflowError:
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_partition_plan(n, nd, align)
        assert e.value.status == 2
        return
    got = Z.zero_partition_plan(n, nd, align)
    assert (got.n, got.padded_n, got.shard_elems, got.pad, got.nd, got.align_elems) == \
        (want.n, want.padded_n, want.shard_elems, want.pad, want.nd, want.align_elems)
    for r in {0, nd // 2, nd - 1, (n // max(want.shard_elems, 1)) % nd}:
        assert Z.zero_shard_range(got, r) == O.shard_range(want, r)


@SETTINGS
@given(n=st.integers(0, 1 << 45), nd=st.integers(1, 4096), stage=st.integers(0, 3),
       pb=st.integers(0, 16), gb=st.integers(0, 16), ob=st.integers(0, 32))
def test_stage_bytes_match_oracle(n, nd, stage, pb, gb, ob):
    plan_c, plan_o = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
    assert tuple(Z.zero_stage_bytes(plan_c, stage, pb, gb, ob)) == \
        tuple(O.stage_bytes_exact(plan_o, stage, pb, gb, ob))


@SETTINGS
@given(n=st.integers(0, 1 << 62), nd=st.integers(1, 1 << 16), stage=st.integers(0, 3),
       pb=st.integers(0, 1 << 20), gb=st.integers(0, 1 << 20))
def test_stage_comm_bytes_match_oracle(n, nd, stage, pb, gb):
    plan_c, plan_o = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
    try:
        want = O.stage_comm_bytes(plan_o, stage, pb, gb)
    except OverflowError:
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_stage_comm_bytes(plan_c, stage, pb, gb)
        assert e.value.status == 2
        return
    assert tuple(Z.zero_stage_comm_bytes(plan_c, stage, pb, gb)) == want


@SETTINGS
@given(n=st.integers(0, 1 << 40), nd=st.integers(1, 1024), usable=st.integers(0, (1 << 64) - 1))
def test_stage_choice_matches_oracle(n, nd, usable):
    plan_c, plan_o = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
    assert Z.zero_choose_stage(plan_c, usable) == O.choose_stage(plan_o, usable)


@SETTINGS
@given(lr=st.floats(0, 10), b1=st.floats(0, 0.9999), b2=st.floats(0, 0.99999),
       eps=st.floats(0, 1), wd=st.floats(0, 1), step=st.integers(1, 1 << 40),
       mode=st.sampled_from(["adamw", "l2"]))
def test_adam_constants_match_oracle(lr, b1, b2, eps, wd, step, mode):
    hp = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, wd_mode=mode, step=step)
    got = Z.zero_adam_derive(Z.adam_hparams(**hp))
    want = O.adam_scalars(O.AdamHParams(**hp))
    for f in ("b1", "b2", "c1", "c2", "ss", "bc", "e", "dec", "w"):
        g, w = np.float32(getattr(got, f)), np.float32(getattr(want, f))
        assert g.view(np.uint32) == w.view(np.uint32) or (np.isnan(g) and np.isnan(w)), (f, g, w)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(lr=st.floats(0, 10), b1=st.floats(0, 0.9999), b2=st.floats(0, 0.99999),
       eps=st.floats(0, 1), wd=st.floats(0, 1), count=st.integers(1, 3000),
       mode=st.sampled_from(["adamw", "l2"]))
def test_adam_constants_table_matches_oracle(lr, b1, b2, eps, wd, count, mode):
    """Every entry t of zero_adam_derive_table is the oracle's constants for step t, bit for bit."""
    hp = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, wd_mode=mode)
    tab = Z.zero_adam_derive_table(Z.adam_hparams(**hp), count)
    got = np.frombuffer(bytes(tab), dtype=np.float32).reshape(count, 9)
    ts = sorted(t for t in {1, 2, count, (count + 1) // 2, 17} if t <= count)
    for t in ts:
        k = O.adam_scalars(O.AdamHParams(**hp, step=t))
        want = np.float32([k.b1, k.b2, k.c1, k.c2, k.ss, k.bc, k.e, k.dec, k.w])
        same = (got[t - 1].view(np.uint32) == want.view(np.uint32)) | (np.isnan(got[t - 1]) & np.isnan(want))
        assert same.all(), (t, got[t - 1], want)


arrays = st.lists(st.tuples(st.integers(0, 1 << 34), st.floats(0, 1), st.integers(0, 5),
                            st.sampled_from([2, 4])), min_size=1, max_size=64)


@SETTINGS
@given(arrays=arrays)
def test_arena_layout_invariants(arrays):
    stagger = {2: 2048, 4: 12288}
    spec = [(n * eb, int(n * f) * eb, g, eb) for n, f, g, eb in arrays]
    offs, total = Z.zero_arena_layout(spec)
    member, end = {}, 0
    for (nbytes, hot, g, eb), off in zip(spec, offs):
        k = member.get(g, 0)
        member[g] = k + 1
        q = 1 << max(22, min(28, (max(nbytes, 1) - 1).bit_length()))   # [4 MiB, 256 MiB]
        assert end <= off < end + q
        assert (off + hot) % q == (k * stagger[eb]) % q
        end = off + nbytes
    assert total == end
