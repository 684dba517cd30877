"""The C-ABI library on the CPU: it loads, exports what the header declares, binds to torch's HIP
runtime, and its host-only entry points match the oracle exactly. Device entry points are only
called with arguments that fail validation (they return before any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import zero_partition_plan_amd as Z

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "zero_shard.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:zero_status|const char\*|uint64_t)\s+(zero_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 9
    L = Z.lib()
    for name in names:
        assert hasattr(L, name), name
    # and the binding exposes the same names
    for name in names:
        assert callable(getattr(Z, name)), name


def test_one_hip_runtime_in_process():
    Z.lib()
    maps = open("/proc/self/maps").read()
    hip = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define ZERO_MAX_REPLICAS (\d+)", text).group(1)) == Z.ZERO_MAX_REPLICAS
    assert "ZERO_SQ_PARTIALS" not in text
    assert ctypes.sizeof(Z.ZeroPlan) == 40 and ctypes.sizeof(Z.ZeroAdamHParams) == 56


@pytest.mark.parametrize("align", (1, 2, 8, 64, 256))
def test_plan_matches_oracle(align):
    for n in list(range(0, 70)) + [299, 1_000_003, 6_738_415_616, 174_604_259_328, (1 << 63) + 5]:
        for nd in (1, 2, 3, 4, 7, 8, 16, 17, 64):
            try:
                want = O.partition_plan(n, nd, align)
            except OverflowError:
                with pytest.raises(Z.ZeroError) as e:
                    Z.zero_partition_plan(n, nd, align)
                assert e.value.status == 2
                continue
            got = Z.zero_partition_plan(n, nd, align)
            assert (got.n, got.padded_n, got.shard_elems, got.pad, got.nd, got.align_elems) == \
                (want.n, want.padded_n, want.shard_elems, want.pad, want.nd, want.align_elems)
            for r in sorted({0, nd // 2, nd - 1}):
                assert Z.zero_shard_range(got, r) == O.shard_range(want, r)


def test_plan_errors():
    for args in ((10, 0, 1), (10, 2, 0)):
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_partition_plan(*args)
        assert e.value.status == 1
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_partition_plan((1 << 64) - 1, 3, 1 << 31)
    assert e.value.status == 2
    p = Z.zero_partition_plan(100, 4)
    with pytest.raises(Z.ZeroError):
        Z.zero_shard_range(p, 4)
    bad = Z.ZeroPlan(100, 101, 25, 1, 4, 1)            # inconsistent: 25 * 4 != 101
    with pytest.raises(Z.ZeroError):
        Z.zero_shard_range(bad, 0)
    assert "rank" in Z.zero_last_error() or "inconsistent" in Z.zero_last_error()


def test_stage_bytes_match_oracle():
    for n, nd in ((1_000_003, 4), (124_356_864, 8), (6_738_415_616, 8), (13_015_864_320, 16)):
        p, op = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
        for stage in range(4):
            for pb, gb, ob in ((2, 2, 12), (2, 4, 12), (4, 4, 8)):
                assert Z.zero_stage_bytes(p, stage, pb, gb, ob) == O.stage_bytes_exact(op, stage, pb, gb, ob)
    with pytest.raises(Z.ZeroError):
        Z.zero_stage_bytes(Z.zero_partition_plan(10, 2), 4)
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_stage_bytes(Z.zero_partition_plan((1 << 62), 1), 0, 2, 2, 12)
    assert e.value.status == 2


def test_stage_comm_bytes_match_oracle():
    for n, nd in ((1_000_003, 4), (124_356_864, 8), (6_738_415_616, 8), (174_604_259_328, 64), (5, 1)):
        p, op = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
        for stage in range(4):
            for pb, gb in ((2, 2), (2, 4), (4, 4), (0, 2)):
                assert Z.zero_stage_comm_bytes(p, stage, pb, gb) == O.stage_comm_bytes(op, stage, pb, gb)
    with pytest.raises(Z.ZeroError):
        Z.zero_stage_comm_bytes(Z.zero_partition_plan(10, 2), 4)
    bad = Z.zero_partition_plan(10, 2)
    bad.pad = 3
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_stage_comm_bytes(bad, 0)
    assert e.value.status == 1 and "inconsistent" in Z.zero_last_error()
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_stage_comm_bytes(Z.zero_partition_plan(1 << 62, 4), 3, 2, 2)
    assert e.value.status == 2


def test_choose_stage_matches_oracle():
    for n in (0, 1, 999, 7_000_000_000, 13_000_000_000, 70_000_000_000, 174_604_259_328):
        for nd in (1, 3, 8, 64):
            for usable in (0, 10**9, 60 * 10**9, 80 * 10**9, 288 * 10**9, (1 << 64) - 1):
                plan_c, plan_o = Z.zero_partition_plan(n, nd), O.partition_plan(n, nd)
                for pb, gb, ob in ((2, 2, 12), (2, 4, 12), (4, 4, 8)):
                    assert Z.zero_choose_stage(plan_c, usable, pb, gb, ob) == \
                        O.choose_stage(plan_o, usable, pb, gb, ob), (n, nd, usable, pb, gb, ob)
    with pytest.raises(Z.ZeroError):
        Z.zero_choose_stage(Z.zero_partition_plan(1 << 62, 1), 0, 8, 8, 8)   # byte overflow


def test_adam_scalars_match_oracle_bitwise():
    rng = np.random.default_rng(9)
    cases = [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t) for t in (1, 2, 11, 1000)]
    for _ in range(200):
        cases.append(dict(lr=float(10 ** rng.uniform(-6, -1)), beta1=float(rng.uniform(0, 0.99)),
                          beta2=float(rng.uniform(0.9, 0.99999)), eps=float(10 ** rng.uniform(-12, -4)),
                          weight_decay=float(rng.uniform(0, 0.3)), step=int(rng.integers(1, 100000))))
    for c in cases:
        got = Z.zero_adam_derive(Z.adam_hparams(**c))
        want = O.adam_scalars(O.AdamHParams(**c))
        for k in ("b1", "b2", "c1", "c2", "ss", "bc", "e", "dec", "w"):
            assert np.float32(getattr(got, k)).view(np.uint32) == getattr(want, k).view(np.uint32), (k, c)


def test_adam_derive_rejects_bad_hparams():
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=-1.0),
                dict(lr=float("nan")), dict(weight_decay=float("inf")), dict(wd_mode=7)):
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_adam_derive(Z.adam_hparams(**bad))
        assert e.value.status == 1


# Device entry points, called only with arguments that fail validation before any HIP call.

def _src(ptrs, dtype=Z.ZERO_BF16):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return Z._GradSrc(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), len(ptrs), dtype), arr


def test_device_entry_points_validate_first():
    L = Z.lib()
    hp = Z.adam_hparams()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    ok_src, k1 = _src([fake])
    # no replicas / too many / NULL replica / unknown dtype
    for src, keep in (_src([]), _src([fake] * 65), _src([fake, 0]), _src([fake], 9)):
        assert L.zero_adam_shard_step(ctypes.byref(src), 100, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                      ctypes.byref(hp), None, 0, None, None) == 1
        assert L.zero_reduce_shard(ctypes.byref(src), 100, fake + 4096, None, None, 1.0, None) == 1
    # NULL state
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, None, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), None, 0, None, None) == 1
    # bad hparams
    bad_hp = Z.adam_hparams(step=0)
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                  ctypes.byref(bad_hp), None, 0, None, None) == 1
    # fp32 output is unsupported; unknown output dtype is invalid
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), fake + 16384, Z.ZERO_F32, None, None) == 3
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), fake + 16384, 5, None, None) == 1
    # aliasing: m overlaps master; out overlaps v; master overlaps a replica
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 4096, fake + 4096 + 396, fake + 12288,
                                  ctypes.byref(hp), None, 0, None, None) == 1
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), fake + 12288 + 100, Z.ZERO_BF16, None, None) == 1
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 100, 1.0, fake + 100, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), None, 0, None, None) == 1
    # size overflow
    assert L.zero_adam_shard_step(ctypes.byref(ok_src), 1 << 62, 1.0, fake + 4096, fake + 8192, fake + 12288,
                                  ctypes.byref(hp), None, 0, None, None) == 2
    # reduce: no output requested; out_grad overlapping a replica
    assert L.zero_reduce_shard(ctypes.byref(ok_src), 100, None, None, None, 1.0, None) == 1
    assert L.zero_reduce_shard(ctypes.byref(ok_src), 100, fake + 8, None, None, 1.0, None) == 1
    # sqnorm: NULL partials or out; out inside partials
    assert L.zero_shard_sqnorm(None, 0, 1.0, None, fake, None) == 1
    assert L.zero_shard_sqnorm(None, 0, 1.0, fake, fake + 8, None) == 1
    assert "overlap" in Z.zero_last_error()


def test_device_scale_entry_points_validate_first():
    L = Z.lib()
    hp = Z.adam_hparams()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    ok_src, k1 = _src([fake])
    step = L.zero_adam_shard_step_dev_scale
    # NULL grad scale (even for n = 0); grad scale inside master or the output
    assert step(ctypes.byref(ok_src), 0, None, None, None, None, ctypes.byref(hp), None, 0, None, None) == 1
    assert "d_grad_scale" in Z.zero_last_error()
    assert step(ctypes.byref(ok_src), 100, fake + 4096 + 8, fake + 4096, fake + 8192, fake + 12288,
                ctypes.byref(hp), None, 0, None, None) == 1
    assert "grad scale" in Z.zero_last_error()
    assert step(ctypes.byref(ok_src), 100, fake + 16384 + 4, fake + 4096, fake + 8192, fake + 12288,
                ctypes.byref(hp), fake + 16384, Z.ZERO_BF16, None, None) == 1
    # the rest is zero_adam_shard_step's validation
    assert step(ctypes.byref(ok_src), 100, fake + 20000, None, fake + 8192, fake + 12288,
                ctypes.byref(hp), None, 0, None, None) == 1
    assert step(ctypes.byref(ok_src), 100, fake + 20000, fake + 4096, fake + 8192, fake + 12288,
                ctypes.byref(Z.adam_hparams(step=0)), None, 0, None, None) == 1
    assert step(ctypes.byref(ok_src), 1 << 62, fake + 20000, fake + 4096, fake + 8192, fake + 12288,
                ctypes.byref(hp), None, 0, None, None) == 2
    # n = 0 with a grad scale pointer: a no-op before any HIP call
    assert step(ctypes.byref(ok_src), 0, fake, None, None, None, ctypes.byref(hp), None, 0, None, None) == 0
    clip = L.zero_clip_scale
    assert clip(None, 1.0, 1e-6, 1.0, fake, None) == 1
    assert clip(fake, 1.0, 1e-6, 1.0, None, None) == 1
    assert clip(fake, 1.0, 1e-6, 1.0, fake + 4, None) == 1          # scale inside the norm
    assert "overlaps" in Z.zero_last_error()
    for mn, eps, inv in ((0.0, 1e-6, 1.0), (-1.0, 1e-6, 1.0), (float("inf"), 1e-6, 1.0),
                         (float("nan"), 1e-6, 1.0), (1.0, -1e-6, 1.0), (1.0, float("nan"), 1.0),
                         (1.0, float("inf"), 1.0), (1.0, 1e-6, 0.0), (1.0, 1e-6, -1.0),
                         (1.0, 1e-6, float("inf"))):
        assert clip(fake, mn, eps, inv, fake + 8, None) == 1, (mn, eps, inv)


def test_derive_table_matches_oracle_per_step():
    for kw in (dict(lr=1e-3, weight_decay=0.01), dict(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6,
                                                      weight_decay=0.1, wd_mode="l2", step=77)):
        hp = Z.adam_hparams(**kw)
        tab = Z.zero_adam_derive_table(hp, 300)
        for t in (1, 2, 3, 10, 11, 299, 300):
            want = O.adam_scalars(O.AdamHParams(**{**kw, "step": t}))
            got = tab[t - 1]
            for f in ("b1", "b2", "c1", "c2", "ss", "bc", "e", "dec", "w"):
                assert np.float32(getattr(got, f)).view(np.uint32) == \
                    np.float32(getattr(want, f)).view(np.uint32), (kw, t, f)
        dev = Z.adam_table(hp, 4, device="cpu")
        assert dev.shape == (4, 9) and float(dev[3, 4]) == tab[3].ss and float(dev[0, 5]) == tab[0].bc
    L = Z.lib()
    out = (Z.ZeroAdamScalars * 2)()
    hp = Z.adam_hparams()
    assert L.zero_adam_derive_table(None, 2, out) == 1
    assert L.zero_adam_derive_table(ctypes.byref(hp), 2, None) == 1
    assert L.zero_adam_derive_table(ctypes.byref(hp), 0, out) == 1
    assert L.zero_adam_derive_table(ctypes.byref(Z.adam_hparams(beta1=1.0)), 2, out) == 1


def test_device_step_entry_point_validates_first():
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    ok_src, k1 = _src([fake])
    step = L.zero_adam_shard_step_dev_t
    gs, tab, t, st = fake + 100000, fake + 200000, fake + 300000, fake + 400000
    P, M, V = fake + 4096, fake + 8192, fake + 12288

    def call(n, gs_, tab_, len_, t_, st_, mode, p, m, v, out=None, odt=0, skip=None):
        return step(ctypes.byref(ok_src), n, gs_, tab_, len_, t_, st_, mode, p, m, v, out, odt, skip, None)

    # NULL grad scale / table / step / status, empty table, unknown wd_mode (even for n = 0)
    assert call(0, None, tab, 4, t, st, 0, None, None, None) == 1
    assert call(0, gs, None, 4, t, st, 0, None, None, None) == 1
    assert call(0, gs, tab, 4, None, st, 0, None, None, None) == 1
    assert call(0, gs, tab, 4, t, None, 0, None, None, None) == 1
    assert "d_status" in Z.zero_last_error()
    assert call(0, gs, tab, 0, t, st, 0, None, None, None) == 1
    assert call(0, gs, tab, 4, t, st, 9, None, None, None) == 1
    # the step inside the table, on the grad scale, on the flag or inside a replica
    assert call(100, gs, tab, 4, tab + 36, st, 0, P, M, V) == 1
    assert call(100, gs, tab, 4, gs, st, 0, P, M, V) == 1
    assert call(100, gs, tab, 4, t, st, 0, P, M, V, skip=t + 4) == 1
    assert "d_step overlaps" in Z.zero_last_error()
    assert call(100, gs, tab, 4, fake + 64, st, 0, P, M, V) == 1
    assert "d_step overlaps replica 0" in Z.zero_last_error()
    # the status word inside any array or word of the call
    for where, what in ((P + 8, "master"), (M, "m"), (V + 396, "v"), (tab + 4, "constants table"),
                        (gs, "grad scale"), (t + 4, "the step"), (fake + 10, "replica 0")):
        assert call(100, gs, tab, 4, t, where, 0, P, M, V) == 1, what
        assert "d_status overlaps" in Z.zero_last_error() and what in Z.zero_last_error(), what
    assert call(100, gs, tab, 4, t, fake + 20000, 0, P, M, V, out=fake + 20000 - 8, odt=Z.ZERO_BF16) == 1
    assert "d_status overlaps out_param" in Z.zero_last_error()
    assert call(100, gs, tab, 4, t, fake + 30000, 0, P, M, V, skip=fake + 30000) == 1
    assert "d_status overlaps the skip flag" in Z.zero_last_error()
    # an output array over the table, the step, the grad scale or the skip flag
    assert call(100, gs, tab, 4, t, st, 0, tab - 8, M, V) == 1
    assert "constants table" in Z.zero_last_error()
    assert call(100, gs, tab, 4, t, st, 0, P, t - 4, V) == 1
    assert call(100, gs, tab, 4, t, st, 0, P, M, V, out=gs - 2, odt=Z.ZERO_BF16) == 1
    assert call(100, gs, tab, 4, t, st, 0, P, M, V, skip=V + 40) == 1
    assert "skip flag" in Z.zero_last_error()
    # zero_adam_shard_step's own checks still apply
    assert call(100, gs, tab, 4, t, st, 0, None, M, V) == 1
    assert call(100, gs, tab, 4, t, st, 0, P, M, V, out=fake + 16384, odt=Z.ZERO_F32) == 3
    assert call(1 << 62, gs, tab, 4, t, st, 0, P, M, V) == 2


def test_flag_words_must_not_alias_arrays():
    """A flag the kernels read (skip) or write (non-finite) lying inside an array the same call
    writes, or a written flag inside a replica, would change under the blocks that start later:
    each such placement is refused before any launch."""
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    hp = Z.adam_hparams()
    src, keep = _src([fake, fake + 8192], Z.ZERO_BF16)
    P, M, V, O = fake + (1 << 20), fake + (2 << 20), fake + (3 << 20), fake + (4 << 20)
    n = 1000
    for skip, what in ((P + 12, "master"), (M, "m"), (V + 3996, "v"), (O + 100, "out_param")):
        assert L.zero_adam_shard_step(ctypes.byref(src), n, 1.0, P, M, V, ctypes.byref(hp), O,
                                      Z.ZERO_BF16, skip, None) == 1, what
        assert "skip flag" in Z.zero_last_error() and what in Z.zero_last_error(), what
    # a skip flag next to the arrays (not inside) is fine up to the launch: n = 0 launches nothing
    assert L.zero_adam_shard_step(ctypes.byref(src), 0, 1.0, P, M, V, ctypes.byref(hp), O,
                                  Z.ZERO_BF16, P - 4, None) == 0
    G, parts = fake + (5 << 20), fake + (6 << 20)
    for flag, what in ((fake + 100, "replica 0"), (fake + 8192 + 1996, "replica 1"), (G + 8, "out_grad"),
                       (parts + 16, "the partials")):
        assert L.zero_reduce_shard(ctypes.byref(src), n, G, flag, parts, 1.0, None) == 1, what
        assert "d_nonfinite overlaps" in Z.zero_last_error() and what in Z.zero_last_error(), what


def test_sq_partials_len():
    # one partial per 256-element tile, then 1024 second-level slots; no wrap-around at the top
    for n, want in ((0, 1024), (1, 1025), (256, 1025), (257, 1026), (813_491_520, 3_177_702 + 1024),
                    (1 << 40, (1 << 32) + 1024), ((1 << 64) - 1, (1 << 56) + 1024)):
        assert Z.zero_sq_partials_len(n) == want, n


def test_zero_length_calls_accept_null_arrays():
    """n = 0 is a no-op that still validates counts, dtypes and hyper-parameters, and returns
    before any HIP call, so it runs on the CPU."""
    L = Z.lib()
    hp = Z.adam_hparams()
    src, keep = _src([0, 0], Z.ZERO_BF16)
    assert L.zero_adam_shard_step(ctypes.byref(src), 0, 1.0, None, None, None, ctypes.byref(hp),
                                  None, 0, None, None) == 0
    assert L.zero_reduce_shard(ctypes.byref(src), 0, None, None, 1 << 40, 1.0, None) == 0
    bad_hp = Z.adam_hparams(step=0)
    assert L.zero_adam_shard_step(ctypes.byref(src), 0, 1.0, None, None, None, ctypes.byref(bad_hp),
                                  None, 0, None, None) == 1
    too_many, keep2 = _src([0] * 65)
    assert L.zero_reduce_shard(ctypes.byref(too_many), 0, None, None, 1 << 40, 1.0, None) == 1


def test_status_strings():
    for s in range(5):
        assert Z.zero_status_str(s)
    assert Z.zero_status_str(99) == "unknown status"


Q = 256 << 20                                   # ZERO_ARENA_GRANULE
QMIN = 4 << 20                                  # ZERO_ARENA_MIN_GRANULE
STAGGER = {2: 2048, 4: 12288}                   # ZERO_ARENA_STAGGER16 / 32


def granule(nbytes):
    """An array's line: its size rounded up to a power of two, within [QMIN, Q]."""
    q = QMIN
    while q < nbytes and q < Q:
        q *= 2
    return q


def test_arena_constants_match_header():
    text = open(HEADER).read()
    assert re.search(r"#define ZERO_ARENA_GRANULE \(256ull << 20\)", text)
    assert re.search(r"#define ZERO_ARENA_MIN_GRANULE \(4ull << 20\)", text)
    assert int(re.search(r"#define ZERO_ARENA_STAGGER16 (\d+)ull", text).group(1)) == STAGGER[2]
    assert int(re.search(r"#define ZERO_ARENA_STAGGER32 (\d+)ull", text).group(1)) == STAGGER[4]
    assert ctypes.sizeof(Z.ZeroArenaArray) == 24


def _check_layout(arrays, offs, total):
    member, end = {}, 0
    for (nbytes, hot, group, eb), off in zip(arrays, offs):
        k = member.get(group, 0)
        member[group] = k + 1
        q = granule(nbytes)
        assert off >= end and off - end < q                  # in order, no overlap, gap < granule
        assert (off + hot) % q == (k * STAGGER[eb]) % q      # hot start: granule line + k * stagger
        assert off % eb == 0 and (off + hot) % 2048 == 0
        end = off + nbytes
    assert total == end


@pytest.mark.parametrize("seed", range(6))
def test_arena_layout_rule(seed):
    rng = np.random.default_rng(seed)
    arrays = []
    for _ in range(int(rng.integers(1, 40))):
        eb = int(rng.choice([2, 4]))
        n = int(rng.integers(0, 1 << int(rng.integers(1, 32))))
        hot = int(rng.integers(0, n + 1)) if n and rng.random() < 0.3 else 0
        arrays.append((n * eb, hot * eb, int(rng.integers(0, 4)) * 977, eb))
    offs, total = Z.zero_arena_layout(arrays)
    _check_layout(arrays, offs, total)


def test_arena_layout_of_the_7b_step():
    """Eight bf16 replica rows and the gathered buffer (walked from rank 0's slot) in one group,
    master/m/v in another: hot starts at 0, 2, .., 16 KiB and 0, 12, 24 KiB past 256 MiB lines."""
    S, P = 842_301_952, 6_738_415_616
    arrays = [(2 * S, 0, 0, 2)] * 8 + [(2 * P, 0, 0, 2)] + [(4 * S, 0, 1, 4)] * 3
    offs, total = Z.zero_arena_layout(arrays)
    _check_layout(arrays, offs, total)
    assert [(o % Q) for o in offs] == [2048 * k for k in range(9)] + [0, 12288, 24576]
    assert total < 2 * P + 11 * 4 * S


def test_arena_layout_errors():
    ok = (1024, 0, 0, 2)
    for bad in [(1024, 0, 0, 3), (1024, 2048, 0, 2), (1023, 0, 0, 2), (1024, 2, 0, 4)]:
        with pytest.raises(Z.ZeroError) as e:
            Z.zero_arena_layout([ok, bad])
        assert e.value.status == 1, bad
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_arena_layout([])
    assert e.value.status == 1
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_arena_layout([ok] * 257)
    assert e.value.status == 1
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_arena_layout([(1 << 63, 0, 0, 2), (1 << 63, 0, 1, 2)])
    assert e.value.status == 2
    L = Z.lib()
    arr = (Z.ZeroArenaArray * 1)(Z.ZeroArenaArray(64, 0, 0, 2))
    out = (ctypes.c_uint64 * 1)()
    tot = ctypes.c_uint64()
    assert L.zero_arena_layout(None, 1, out, ctypes.byref(tot)) == 1
    assert L.zero_arena_layout(arr, 1, None, ctypes.byref(tot)) == 1
    assert L.zero_arena_layout(arr, 1, out, None) == 1


def test_arena_views_on_host_memory():
    import torch
    specs = [("a", 1000, torch.bfloat16, 0, 0), ("b", 3000, torch.float16, 0, 17),
             ("c", 513, torch.float32, 1, 0), ("d", 7, torch.float32, 1, 0)]
    storage, views = Z.arena(specs, device="cpu")
    base = storage.data_ptr()
    offs, total = Z.zero_arena_layout([(n * t.element_size(), h * t.element_size(), g, t.element_size())
                                       for (_, n, t, g, h) in [(s[0], s[1], torch.empty(0, dtype=s[2]),
                                                                s[3], s[4]) for s in specs]])
    assert storage.numel() == total
    for (name, n, dt, _, _), off in zip(specs, offs):
        v = views[name]
        assert v.dtype == dt and v.shape == (n,) and v.data_ptr() - base == off
    for i, (name, *_rest) in enumerate(specs):  # the views do not overlap
        views[name].fill_(float(i + 1))
    for i, (name, *_rest) in enumerate(specs):
        assert (views[name] == float(i + 1)).all(), name


def test_error_messages_are_per_thread():
    """zero_last_error() is thread-local: threads that fail in different ways at the same time each
    read their own message (ctypes releases the GIL for the call, so the calls overlap)."""
    import threading

    L = Z.lib()
    results, start = {}, threading.Barrier(8)

    def worker(k):
        plan = Z.ZeroPlan()
        start.wait()
        seen = set()
        for _ in range(2000):
            if k % 2:
                assert L.zero_partition_plan(5, 0, 1, ctypes.byref(plan)) == 1
                want = "nd must be >= 1"
            else:
                assert L.zero_partition_plan(5, 1, 0, ctypes.byref(plan)) == 1
                want = "align_elems must be >= 1"
            msg = L.zero_last_error().decode()
            seen.add(want in msg)
        results[k] = seen

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(v == {True} for v in results.values()), results


def test_arrays_off_natural_alignment_are_refused():
    """Any element offset is accepted, but an array must be aligned to its own element size (the
    hardware drops the low address bits of word-sized accesses): a float pointer one byte off, or a
    16-bit one an odd byte off, is refused before any launch."""
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    hp = Z.adam_hparams()
    P, M, V, O = fake + (1 << 20), fake + (2 << 20), fake + (3 << 20), fake + (4 << 20)
    good16, k1 = _src([fake + 2, fake + 8194], Z.ZERO_BF16)     # odd elements: fine
    bad16, k2 = _src([fake, fake + 8193], Z.ZERO_BF16)
    bad32, k3 = _src([fake + 6], Z.ZERO_F32)
    n = 1000
    for src, args, what in ((bad16, (P, M, V, O), "replica 1"), (bad32, (P, M, V, O), "replica 0"),
                            (good16, (P + 1, M, V, O), "master"), (good16, (P, M + 2, V, O), "master"),
                            (good16, (P, M, V + 3, O), "master"), (good16, (P, M, V, O + 1), "master")):
        assert L.zero_adam_shard_step(ctypes.byref(src), n, 1.0, *args[:3], ctypes.byref(hp), args[3],
                                      Z.ZERO_BF16, None, None) == 1, what
        assert "not aligned" in Z.zero_last_error(), what
    G, parts = fake + (5 << 20), fake + (6 << 20)
    assert L.zero_reduce_shard(ctypes.byref(bad16), n, G, None, None, 1.0, None) == 1
    assert L.zero_reduce_shard(ctypes.byref(good16), n, G + 2, None, None, 1.0, None) == 1
    assert L.zero_reduce_shard(ctypes.byref(good16), n, None, None, parts + 4, 1.0, None) == 1
    assert L.zero_shard_sqnorm(G + 1, n, 1.0, parts, parts - 8, None) == 1
    assert "not aligned" in Z.zero_last_error()


def test_static_reduce_checks_its_reach_first():
    """The no-allocation reduce refuses a shard its scratch cannot cover (only when a norm is
    asked for), and checks aliasing and alignment, all before any device work."""
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    src, keep = _src([fake], Z.ZERO_F16)
    sq, G = fake + (64 << 30), fake + (128 << 30)
    big = Z.ZERO_STATIC_MAX_ELEMS + 1
    assert Z.ZERO_STATIC_MAX_ELEMS == 1_073_479_680
    assert L.zero_reduce_shard_static(ctypes.byref(src), big, None, None, 1.0, sq, None) == 1
    assert "exceeds" in Z.zero_last_error()
    assert L.zero_reduce_shard_static(ctypes.byref(src), 100, None, None, 1.0, None, None) == 1
    assert "no output" in Z.zero_last_error()
    assert L.zero_reduce_shard_static(ctypes.byref(src), 100, None, None, 1.0, fake + 40, None) == 1
    assert "d_sq overlaps replica 0" in Z.zero_last_error()
    assert L.zero_reduce_shard_static(ctypes.byref(src), 100, G, None, 1.0, G + 8, None) == 1
    assert L.zero_reduce_shard_static(ctypes.byref(src), 100, None, sq, 1.0, sq, None) == 1
    assert "d_nonfinite overlaps d_sq" in Z.zero_last_error()
    assert L.zero_reduce_shard_static(ctypes.byref(src), 100, None, None, 1.0, sq + 4, None) == 1
    assert "not aligned" in Z.zero_last_error()
    text = open(HEADER).read()
    assert "#define ZERO_STATIC_SQ_PARTIALS (4u << 20)" in text


def test_offload_step_needs_four_distinct_events():
    """zero_offload_step creates no HIP objects: its four events come with the caller's staging,
    and a NULL or repeated one is refused before any device work."""
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    hp = Z.adam_hparams()
    src, keep = _src([fake], Z.ZERO_BF16)
    h = (ctypes.c_float * 64)()
    hm, hv = (ctypes.c_float * 64)(), (ctypes.c_float * 64)()
    ev = [fake + 0x100, fake + 0x200, fake + 0x300, fake + 0x400]

    def bufs(events):
        return Z.ZeroOffloadBuffers(fake + (1 << 20), fake + (2 << 20), fake + (3 << 20), 16, 1, 0, None,
                                    (ctypes.c_void_p * 4)(*events))

    for events, what in (([None] + ev[1:], "event 0 is NULL"), (ev[:3] + [None], "event 3 is NULL"),
                         ([ev[0], ev[1], ev[0], ev[3]], "events 0 and 2 are the same")):
        b = bufs(events)
        assert L.zero_offload_step(ctypes.byref(src), 64, 1.0, h, hm, hv, ctypes.byref(hp), fake + (4 << 20),
                                   Z.ZERO_BF16, ctypes.byref(b), None) == 1, what
        assert what in Z.zero_last_error(), (what, Z.zero_last_error())
    assert ctypes.sizeof(Z.ZeroOffloadBuffers) == 8 * 3 + 8 + 4 + 4 + 8 + 4 * 8


def test_offload_direct_staging_checks():
    """With no device staging (d_grad NULL) the reduce kernel writes the pinned host chunks
    itself, so those are what is checked against the slot and the replicas; a NULL h_grad is
    still refused. All refused before any device work."""
    L = Z.lib()
    fake = 1 << 40                                   # never dereferenced: every call below is invalid
    hp = Z.adam_hparams()
    src, keep = _src([fake], Z.ZERO_BF16)
    h = (ctypes.c_float * 64)()
    hm, hv = (ctypes.c_float * 64)(), (ctypes.c_float * 64)()
    ev = (ctypes.c_void_p * 4)(fake + 0x100, fake + 0x200, fake + 0x300, fake + 0x400)
    slot = fake + (4 << 20)

    def call(h_grad, out=slot):
        b = Z.ZeroOffloadBuffers(None, h_grad, fake + (3 << 20), 16, 1, 0, None, ev)
        return L.zero_offload_step(ctypes.byref(src), 64, 1.0, h, hm, hv, ctypes.byref(hp), out,
                                   Z.ZERO_BF16, ctypes.byref(b), None)

    assert call(None) == 1 and "incomplete staging buffers" in Z.zero_last_error()
    assert call(slot + 100) == 1 and "the slot overlaps the gradient staging" in Z.zero_last_error()
    assert call(fake + 64) == 1 and "the gradient staging overlaps replica 0" in Z.zero_last_error()
