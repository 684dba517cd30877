"""GPU parity of the fused sharded step and the reduce / squared-norm passes, at sizes the oracle
finishes in seconds. Every comparison of fp32 state and 16-bit output is bit for bit (the library
and the oracle evaluate the same fp32 operation order with IEEE rounding); the squared norm, an
fp64 sum in a different order, is held to 1e-10 relative."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import (DEV, assert_bits_equal, assert_bits_equal_nan, banner, bits16, bits32, dev_f32,
                      dev_rep, empty16, f32_bits)
from cast_check import check_cast_slice
from workloads import WORKLOADS
from workloads import host as H
from workloads.extremes import EXTREME_CASES, f16_all_patterns, f32_patterns, mixed_state

pytestmark = pytest.mark.gpu

_T16 = {"bf16": torch.bfloat16, "f16": torch.float16}
TILE = 256  # elements per tile of both the reduce and the Adam kernel (64 threads x 4)


def _reps_np(rng, R, n, dtype, std=1e-3, valid=None):
    x = (rng.standard_normal((R, n)).astype(np.float32) * np.float32(std))
    if valid is not None:
        x[:, valid:] = 0
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return (x * np.float32(64.0)).astype(np.float16).view(np.uint16)


def _run_step(reps_np, dtype, n, master, m, v, hp_kw, out_dtype, grad_scale=1.0, offsets=(0, 0, 0, 0, 0)):
    """Run the kernel on device copies placed at element offsets (rep, master, m, v, out) to reach
    the aligned and misaligned paths; return (master, m, v, out16 or None) as numpy bit arrays."""
    orep, op, om, ov, oo = offsets
    R = reps_np.shape[0]
    d_reps = [dev_rep(np.concatenate([np.zeros(orep, reps_np.dtype), r]), dtype)[orep:] for r in reps_np]
    d_p = dev_f32(np.concatenate([np.zeros(op, np.float32), master]))[op:]
    d_m = dev_f32(np.concatenate([np.zeros(om, np.float32), m]))[om:]
    d_v = dev_f32(np.concatenate([np.zeros(ov, np.float32), v]))[ov:]
    d_o = None
    if out_dtype is not None:
        d_o = empty16(n + oo + 5, out_dtype, fill=-3.0)
    Z.zero_adam_shard_step(d_reps, n, grad_scale, d_p, d_m, d_v, Z.adam_hparams(**hp_kw),
                           out=None if d_o is None else d_o[oo:oo + n])
    torch.cuda.synchronize()
    out = None
    if d_o is not None:
        full = bits16(d_o)
        canary = O.cast_bf16_rne(np.float32([-3.0]))[0] if out_dtype == "bf16" else O.cast_fp16_rne(np.float32([-3.0]))[0]
        assert (full[:oo] == canary).all() and (full[oo + n:] == canary).all(), "write outside the slot"
        out = full[oo:oo + n]
    return bits32(d_p), bits32(d_m), bits32(d_v), out


def _check_step(reps_np, dtype, n, hp_kw, out_dtype, rng, grad_scale=1.0, offsets=(0, 0, 0, 0, 0),
                warm=True):
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32) if warm else np.zeros(n, np.float32)
    got = _run_step(reps_np, dtype, n, master, m, v, hp_kw, out_dtype, grad_scale, offsets)
    p2, m2, v2, o2 = O.sharded_step(list(reps_np), dtype, grad_scale, master, m, v,
                                    O.AdamHParams(**hp_kw), out_dtype)
    assert_bits_equal(got[0], f32_bits(p2), "master")
    assert_bits_equal(got[1], f32_bits(m2), "m")
    assert_bits_equal(got[2], f32_bits(v2), "v")
    if out_dtype is not None:
        assert_bits_equal(got[3], o2, "out")


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=3)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 8, 9, 16, 17, 64])
def test_step_replica_counts_and_dtypes(dtype, R):
    n = 3 * TILE + 1234                      # several full tiles and a ragged tail
    banner(f"step dtype={dtype} R={R} n={n}")
    rng = np.random.default_rng(100 + R)
    _check_step(_reps_np(rng, R, n, dtype), dtype, n, HP, "bf16", rng)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16", None])
@pytest.mark.parametrize("mode", ["adamw", "l2"])
def test_step_outputs_and_decay_modes(out_dtype, mode):
    n = 5 * TILE + 77
    banner(f"step out={out_dtype} mode={mode}")
    rng = np.random.default_rng(7)
    hp = {**HP, "wd_mode": mode, "weight_decay": 0.05, "step": 1}
    _check_step(_reps_np(rng, 8, n, "bf16"), "bf16", n, hp, out_dtype, rng, grad_scale=0.125)


@pytest.mark.parametrize("offsets", [(1, 0, 0, 0, 0), (0, 1, 0, 0, 0), (0, 0, 2, 0, 0),
                                     (0, 0, 0, 3, 0), (0, 0, 0, 0, 1), (3, 1, 2, 3, 5)])
def test_step_misaligned_arrays(offsets):
    n = 2 * TILE + 999
    banner(f"step misaligned offsets={offsets}")
    rng = np.random.default_rng(sum(offsets))
    _check_step(_reps_np(rng, 3, n, "bf16"), "bf16", n, HP, "bf16", rng, offsets=offsets)


@pytest.mark.parametrize("rdt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("R", [5, 8, 16, 64])
@pytest.mark.parametrize("out_off", [0, 1, 2, 3])
def test_step_replica_and_slot_phases(rdt, R, out_off):
    """Replica k placed k elements into its buffer (16-bit replicas then alternate between starting
    on a 4-byte word and 2 bytes past one), master/m/v 1, 2 and 3 elements in (off 16 bytes), and
    the 16-bit slot at each offset mod 4, over several tiles and a ragged tail: every result bit for
    bit against the oracle, and no byte written outside the slot (its first and last elements sit
    next to the canaries)."""
    n = 9 * TILE + 77
    banner(f"step phases rdt={rdt} R={R} out_off={out_off}")
    rng = np.random.default_rng(1000 * R + out_off)
    reps = _reps_np(rng, R, n, rdt)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    d_reps = [dev_rep(np.concatenate([np.zeros(k % 4, r.dtype), r]), rdt)[k % 4:] for k, r in enumerate(reps)]
    d_p = dev_f32(np.concatenate([np.zeros(1, np.float32), master]))[1:]
    d_m = dev_f32(np.concatenate([np.zeros(2, np.float32), m]))[2:]
    d_v = dev_f32(np.concatenate([np.zeros(3, np.float32), v]))[3:]
    for odt in ("bf16", "f16"):
        p, mm, vv = d_p.clone(), d_m.clone(), d_v.clone()
        full = empty16(n + out_off + 5, odt, fill=-3.0)
        Z.zero_adam_shard_step(d_reps, n, 0.5, p, mm, vv, Z.adam_hparams(**HP), out=full[out_off:out_off + n])
        torch.cuda.synchronize()
        wp, wm, wv, wo = O.sharded_step(list(reps), rdt, 0.5, master, m, v, O.AdamHParams(**HP), odt)
        assert_bits_equal(bits32(p), f32_bits(wp), f"{odt} master")
        assert_bits_equal(bits32(mm), f32_bits(wm), f"{odt} m")
        assert_bits_equal(bits32(vv), f32_bits(wv), f"{odt} v")
        got = bits16(full)
        canary = (O.cast_bf16_rne if odt == "bf16" else O.cast_fp16_rne)(np.float32([-3.0]))[0]
        assert (got[:out_off] == canary).all() and (got[out_off + n:] == canary).all(), "write outside the slot"
        assert_bits_equal(got[out_off:out_off + n], wo, f"{odt} slot")


@pytest.mark.parametrize("rdt", ["bf16", "f16"])
@pytest.mark.parametrize("R", [3, 16, 64])
def test_reduce_replica_phases(rdt, R):
    """The reduce pass with replicas at mixed phases (replica k, k elements into its buffer) and the
    gradient 1 element in: gradient, flag and every per-tile partial bit-equal to the same pass on
    aligned copies, and the gradient bit-equal to the oracle."""
    n = 11 * TILE + 45
    banner(f"reduce phases rdt={rdt} R={R}")
    rng = np.random.default_rng(77 + R)
    reps = _reps_np(rng, R, n, rdt)
    runs = []
    for shifted in (False, True):
        d_reps = [dev_rep(np.concatenate([np.zeros(k % 4 if shifted else 0, r.dtype), r]), rdt)[(k % 4 if shifted else 0):]
                  for k, r in enumerate(reps)]
        g_buf = torch.empty(n + 1, device=DEV)
        g = g_buf[1:] if shifted else g_buf[:n]
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
        Z.zero_reduce_shard(d_reps, n, g, flag, parts, 2.0 ** -6)
        torch.cuda.synchronize()
        runs.append((bits32(g), int(flag.item()), parts.cpu().numpy()[:math.ceil(n / TILE)].copy()))
    assert_bits_equal(runs[1][0], runs[0][0], "gradient")
    assert runs[0][1] == runs[1][1] == 0
    assert np.array_equal(runs[0][2], runs[1][2])
    assert_bits_equal(runs[0][0], f32_bits(O.replica_sum(list(reps), rdt)), "gradient vs oracle")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 1023, TILE - 1, TILE, TILE + 1])
def test_step_small_and_edge_sizes(n):
    banner(f"step n={n}")
    rng = np.random.default_rng(n)
    _check_step(_reps_np(rng, 4, n, "f16"), "f16", n, HP, "f16", rng)


def test_step_n_zero_is_a_no_op():
    d_p = dev_f32(np.ones(16, np.float32))
    d_m = torch.zeros(16, device=DEV)
    d_v = torch.zeros(16, device=DEV)
    rep = dev_rep(np.ones(16, np.float32), "f32")
    Z.zero_adam_shard_step([rep], 0, 1.0, d_p, d_m, d_v, Z.adam_hparams())
    torch.cuda.synchronize()
    assert (d_p.cpu().numpy() == 1).all() and not d_m.any() and not d_v.any()


def test_tiny_workload_all_ranks_three_steps():
    """The tiny workload: N = 1,000,003 over 4 ranks (one padding element), one fp32 gradient,
    Adam 3 steps; every rank works on slices of shared flat buffers, so ranks 1-3 see element
    offsets that are not 16-byte aligned. Results are gathered into one 16-bit buffer and compared
    with the oracle's unsharded update, bit for bit, for both output formats."""
    w = WORKLOADS["tiny"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    S, P = plan.shard_elems, plan.padded_n
    flat = H.flat_inputs(w, P)
    for out_dtype in w.out_dtypes:
        banner(f"tiny workload out={out_dtype}")
        d_p = dev_f32(flat["master"])
        d_m = torch.zeros(P, device=DEV)
        d_v = torch.zeros(P, device=DEV)
        d_g = dev_f32(flat["grad"])
        d_out = empty16(P, out_dtype, fill=0.0)
        p, m, v = flat["master"], np.zeros(P, np.float32), np.zeros(P, np.float32)
        for t in range(1, w.steps + 1):
            hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            for r in range(w.nd):
                b, _ = Z.zero_shard_range(plan, r)
                Z.zero_adam_shard_step([d_g[b:b + S]], S, 1.0, d_p[b:b + S], d_m[b:b + S], d_v[b:b + S],
                                       Z.adam_hparams(**hp), out=d_out[b:b + S])
            torch.cuda.synchronize()
            p, m, v, o = O.unsharded_step(flat["grad"], p, m, v, O.AdamHParams(**hp), out_dtype=out_dtype)
            assert_bits_equal(bits32(d_p), f32_bits(p), f"master step {t}")
            assert_bits_equal(bits32(d_m), f32_bits(m), f"m step {t}")
            assert_bits_equal(bits32(d_v), f32_bits(v), f"v step {t}")
            assert_bits_equal(bits16(d_out), o, f"gathered params step {t}")
        assert bits32(d_p)[w.n:].tolist() == [0] * plan.pad      # padding stays 0


def test_cast_edges_through_the_kernel():
    """Zero gradient on zero state with wd = 0 leaves p unchanged, so the slot receives the cast of
    arbitrary fp32 patterns: ties, subnormals, overflow, infinities, signed zeros."""
    rng = np.random.default_rng(21)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, 300_000, dtype=np.uint64).astype(np.uint32)])
    x = pats.view(np.float32)
    x = x[~np.isnan(x)].copy()
    n = x.size
    zero = np.zeros(n, np.float32)
    for out_dtype, cast in (("bf16", O.cast_bf16_rne), ("f16", O.cast_fp16_rne)):
        banner(f"cast edges {out_dtype} n={n}")
        got = _run_step(np.zeros((1, n), np.float32), "f32", n, x, zero, zero,
                        dict(lr=1e-3, weight_decay=0.0, step=1), out_dtype)
        assert_bits_equal(got[0], f32_bits(x), "master unchanged")
        assert_bits_equal(got[3], cast(x), f"cast {out_dtype}")


def test_cast_of_every_fp32_pattern_through_the_kernel():
    """All 2^32 fp32 patterns as the master copy, in chunks of 2^28, through the fused update with
    zero gradient, zero state and wd = 0 (so p is unchanged up to quieting a NaN) into both 16-bit
    outputs: every non-NaN pattern's cast equals the oracle's bit for bit, and every NaN stays a
    NaN (its payload bits are not the oracle's to fix). The host comparison runs on 16 threads."""
    from concurrent.futures import ThreadPoolExecutor
    chunk, sub = 1 << 28, 1 << 24
    zeros = torch.zeros(chunk, device=DEV)
    m, v = torch.zeros(chunk, device=DEV), torch.zeros(chunk, device=DEV)
    outs = {dt: torch.empty(chunk, dtype=_T16[dt], device=DEV) for dt in ("bf16", "f16")}
    hp = Z.adam_hparams(lr=1e-3, weight_decay=0.0, step=1)
    with ThreadPoolExecutor(16) as pool:
        for c in range(1 << 4):
            banner(f"cast of every fp32 pattern: chunk {c} of 16")
            lo = c * chunk
            signed_lo = lo - (1 << 32) if lo >= 1 << 31 else lo   # each chunk lies in one half
            d_p = torch.arange(signed_lo, signed_lo + chunk, dtype=torch.int64, device=DEV)
            d_p = d_p.to(torch.int32).view(torch.float32)
            for out in outs.values():
                Z.zero_adam_shard_step([zeros], chunk, 1.0, d_p, m, v, hp, out=out)
            got = {dt: bits16(out) for dt, out in outs.items()}
            got_p = bits32(d_p)
            jobs = [pool.submit(check_cast_slice, lo + a, {dt: g[a:a + sub] for dt, g in got.items()},
                                got_p[a:a + sub]) for a in range(0, chunk, sub)]
            errors = [e for e in (j.result() for j in jobs) if e]
            assert not errors, errors[0]
            del d_p


def test_skip_flag():
    n = 3 * TILE + 5
    rng = np.random.default_rng(3)
    reps = _reps_np(rng, 2, n, "bf16")
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    d_p, d_m, d_v = dev_f32(master), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    d_o = empty16(n, "bf16", fill=5.0)
    d_r = [dev_rep(r, "bf16") for r in reps]
    skip = torch.ones(1, dtype=torch.int32, device=DEV)
    Z.zero_adam_shard_step(d_r, n, 1.0, d_p, d_m, d_v, Z.adam_hparams(), out=d_o, skip=skip)
    torch.cuda.synchronize()
    assert_bits_equal(bits32(d_p), f32_bits(master), "skipped master")
    assert not d_m.any() and not d_v.any() and (d_o == 5.0).all()
    skip.zero_()
    Z.zero_adam_shard_step(d_r, n, 1.0, d_p, d_m, d_v, Z.adam_hparams(), out=d_o, skip=skip)
    torch.cuda.synchronize()
    p2, _, _, o2 = O.sharded_step(list(reps), "bf16", 1.0, master, np.zeros(n, np.float32),
                                  np.zeros(n, np.float32), O.AdamHParams(), "bf16")
    assert_bits_equal(bits32(d_p), f32_bits(p2), "stepped master")
    assert_bits_equal(bits16(d_o), o2, "stepped out")


def test_repeat_runs_are_bitwise_identical():
    n = 7 * TILE + 11
    rng = np.random.default_rng(4)
    reps = _reps_np(rng, 8, n, "bf16")
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z = np.zeros(n, np.float32)
    a = _run_step(reps, "bf16", n, master, z, z, HP, "bf16")
    b = _run_step(reps, "bf16", n, master, z, z, HP, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------------ reduce and squared norm

def _reduce(reps_np, dtype, n, sq_scale=1.0, want_grad=True, offset=0):
    d_r = [dev_rep(np.concatenate([np.zeros(offset, reps_np.dtype), r]), dtype)[offset:] for r in reps_np]
    d_g = torch.full((n + offset,), 7.0, device=DEV)[offset:] if want_grad else None
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = torch.full((Z.zero_sq_partials_len(n),), 9.0, dtype=torch.float64, device=DEV)
    out = torch.zeros(1, dtype=torch.float64, device=DEV)
    Z.zero_reduce_shard(d_r, n, d_g, flag, parts, sq_scale)
    Z.zero_shard_sqnorm(None, n, sq_scale, parts, out)
    torch.cuda.synchronize()
    return (None if d_g is None else bits32(d_g)), int(flag.item()), float(out.item()), parts.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("R", [1, 3, 8, 16, 64])
def test_reduce_matches_oracle(dtype, R):
    n = 9 * TILE + 333
    banner(f"reduce dtype={dtype} R={R}")
    rng = np.random.default_rng(200 + R)
    reps = _reps_np(rng, R, n, dtype)
    g, flag, sq, _ = _reduce(reps, dtype, n, sq_scale=2.0 ** -6)
    acc = O.replica_sum(list(reps), dtype)
    assert_bits_equal(g, f32_bits(acc), "reduced grad")
    assert flag == 0
    assert sq == pytest.approx(O.shard_sqnorm(acc, 2.0 ** -6), rel=1e-10, abs=0)


@pytest.mark.parametrize("n", [1, 5, TILE - 1, TILE + 3, 20000 * TILE + 17])
def test_reduce_sizes_and_misalignment(n):
    """A replica on a 4-byte word and one 2 bytes past it (the word-realigning loads): the
    gradient, the per-tile partials and the norm must agree bit for bit between the two."""
    banner(f"reduce n={n}")
    rng = np.random.default_rng(n % 1000)
    reps = _reps_np(rng, 2, n, "bf16")
    acc = O.replica_sum(list(reps), "bf16")
    seen = []
    for offset in (0, 1):
        g, flag, sq, parts = _reduce(reps, "bf16", n, offset=offset)
        assert_bits_equal(g, f32_bits(acc), f"reduced grad offset {offset}")
        assert sq == pytest.approx(O.shard_sqnorm(acc), rel=1e-10, abs=0)
        seen.append((sq, parts[:-(1024)].copy()))
    assert seen[0][0] == seen[1][0]
    assert np.array_equal(seen[0][1], seen[1][1])


def test_reduce_per_tile_partials():
    """Partial t is the squared norm of tile t alone (elements [256t, 256t + 256))."""
    n = 37 * TILE + 101
    rng = np.random.default_rng(77)
    reps = _reps_np(rng, 8, n, "f16")
    acc = O.replica_sum(list(reps), "f16")
    _, _, sq, parts = _reduce(reps, "f16", n, sq_scale=2.0 ** -6)
    ntiles = -(-n // TILE)
    assert Z.zero_sq_partials_len(n) == ntiles + 1024
    for t in range(ntiles):
        want = O.shard_sqnorm(acc[t * TILE:(t + 1) * TILE], 2.0 ** -6)
        assert parts[t] == pytest.approx(want, rel=1e-12, abs=0), t
    assert sq == pytest.approx(math.fsum(parts[:ntiles].tolist()), rel=1e-13, abs=0)


def test_reduce_zero_size():
    reps = np.zeros((1, 4), np.float32)
    _, flag, sq, parts = _reduce(reps, "f32", 0)
    assert sq == 0.0 and flag == 0
    assert (parts == 9.0).all()                  # n = 0 writes no partial


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_reduce_flags_nonfinite(bad):
    n = 4 * TILE + 9
    rng = np.random.default_rng(5)
    reps = _reps_np(rng, 3, n, "f32")
    for pos in (0, 2 * TILE + 17, n - 1):           # vector tile and ragged tail
        r = reps.copy()
        r[1, pos] = bad
        _, flag, _, _ = _reduce(r, "f32", n, want_grad=False)
        assert flag == 1
    # +inf and -inf in two replicas sum to NaN: still flagged
    r = reps.copy()
    r[0, 5], r[2, 5] = np.inf, -np.inf
    assert _reduce(r, "f32", n)[1] == 1


def test_reduce_is_deterministic():
    n = 12000 * TILE + 3
    rng = np.random.default_rng(6)
    reps = _reps_np(rng, 4, n, "f16")
    a = _reduce(reps, "f16", n, sq_scale=2.0 ** -16)
    b = _reduce(reps, "f16", n, sq_scale=2.0 ** -16)
    assert np.array_equal(a[0], b[0]) and a[2] == b[2] and np.array_equal(a[3], b[3])


def test_sqnorm_from_fp32_grad():
    for n in (1, 1000, 77 * TILE + 5):
        rng = np.random.default_rng(n)
        g = (rng.standard_normal(n) * 3).astype(np.float32)
        parts = torch.zeros(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
        out = torch.zeros(1, dtype=torch.float64, device=DEV)
        Z.zero_shard_sqnorm(dev_f32(g), n, 0.5, parts, out)
        torch.cuda.synchronize()
        assert float(out.item()) == pytest.approx(O.shard_sqnorm(g, 0.5), rel=1e-10, abs=0)


# ------------------------------------------------------------------ two-pass clip / overflow path

def _two_pass(reps_np, n, master, loss_scale, max_norm, hp_kw, device_scale):
    """reduce (grad, flag, partials) -> sqnorm -> clip scale -> step with skip flag. The clip scale
    is formed on the host from the read-back norm, or on the device (zero_clip_scale feeding
    zero_adam_shard_step_dev_scale, nothing read back before the update)."""
    d_r = [dev_rep(r, "f16") for r in reps_np]
    d_g = torch.empty(n, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    Z.zero_reduce_shard(d_r, n, d_g, flag, parts, 1.0 / loss_scale)
    Z.zero_shard_sqnorm(None, n, 1.0 / loss_scale, parts, sq)
    d_p, d_m, d_v = dev_f32(master), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    d_o = empty16(n, "f16", fill=0.0)
    hp = Z.adam_hparams(**hp_kw)
    if device_scale:
        d_gs = torch.full((1,), float("nan"), device=DEV)
        Z.zero_clip_scale(sq, max_norm, 1e-6, 1.0 / loss_scale, d_gs)
        Z.zero_adam_shard_step_dev_scale([d_g], n, d_gs, d_p, d_m, d_v, hp, out=d_o, skip=flag)
        torch.cuda.synchronize()
        flag_h, sq_h, gs = int(flag.item()), float(sq.item()), float(d_gs.item())
    else:
        flag_h, sq_h = int(flag.item()), float(sq.item())
        coef = O.clip_coefficient(sq_h, max_norm) if flag_h == 0 else 1.0
        gs = float(np.float32(coef / loss_scale))
        Z.zero_adam_shard_step([d_g], n, gs, d_p, d_m, d_v, hp, out=d_o, skip=flag)
        torch.cuda.synchronize()
    return flag_h, sq_h, gs, bits32(d_p), bits32(d_m), bits32(d_v), bits16(d_o)


@pytest.mark.parametrize("device_scale", [False, True])
@pytest.mark.parametrize("inject", [False, True])
def test_two_pass_clip_and_overflow_skip(inject, device_scale):
    """fp16 replicas holding grad * 2^16: unscale, squared norm, clip coefficient (host or device),
    AdamW; with an injected +inf the whole step is skipped and the state stays bit-identical."""
    n, R, ls = 6 * TILE + 321, 16, 65536.0
    rng = np.random.default_rng(31)
    x = rng.standard_normal((R, n)).astype(np.float32) * np.float32(1e-4)
    reps = (x * np.float32(ls)).astype(np.float16).view(np.uint16)
    if inject:
        reps[5, 1234] = 0x7C00
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(lr=1e-3, weight_decay=0.01, step=1)
    flag, sq, gs, p, m, v, o = _two_pass(reps, n, master, ls, 0.01, hp, device_scale)
    acc = O.replica_sum(list(reps), "f16")
    assert flag == int(O.nonfinite_flag(acc))
    if inject:
        assert_bits_equal(p, f32_bits(master), "skipped master")
        assert not m.any() and not v.any() and not o.any()
        return
    want_sq = O.shard_sqnorm(acc, 1.0 / ls)
    assert sq == pytest.approx(want_sq, rel=1e-10, abs=0)
    coef = O.clip_coefficient(want_sq, 0.01)
    assert coef < 1.0                                   # clipping is active in this case
    # the scale the pipeline used agrees with the oracle's to within one fp32 ulp; the update is
    # then checked bit for bit with that same scale
    want_gs = np.float32(coef / ls)
    assert abs(np.float32(gs) - want_gs) <= np.spacing(want_gs)
    if device_scale:                                    # from the device's own norm, exactly
        assert np.float32(gs) == np.float32(O.clip_coefficient(sq, 0.01) / ls)
    p2, m2, v2, o2 = O.sharded_step([acc], "f32", gs, master, np.zeros(n, np.float32),
                                    np.zeros(n, np.float32), O.AdamHParams(**hp), "f16")
    assert_bits_equal(p, f32_bits(p2), "master")
    assert_bits_equal(m, f32_bits(m2), "m")
    assert_bits_equal(v, f32_bits(v2), "v")
    assert_bits_equal(o, o2, "fp16 params")


def test_clip_scale_matches_fp64_formula():
    """zero_clip_scale over norms from 0 and subnormals to huge, inf and NaN, and several max_norm,
    eps and loss scales: the device's fp32 scale equals the oracle's clip coefficient, formed in
    correctly rounded fp64 and rounded once to fp32, bit for bit."""
    rng = np.random.default_rng(77)
    sqs = [0.0, 5e-324, 2.2e-308, 1e-300, 1e-12, 1e-4, 0.25, 1.0, 4.0, 1e4, 1e300, 1.7e308,
           float("inf"), float("nan")]
    sqs += list(10.0 ** rng.uniform(-300, 300, 60)) + list(rng.uniform(0, 4, 40))
    cases = [(mn, eps, inv) for mn in (1.0, 0.01, 3.7) for eps in (1e-6, 0.0)
             for inv in (2.0 ** -16, 1.0, 1.0 / 3.0)]
    d_sq = torch.tensor(sqs, dtype=torch.float64, device=DEV)
    for mn, eps, inv in cases:
        out = torch.full((len(sqs),), float("nan"), device=DEV)
        for i in range(len(sqs)):
            Z.zero_clip_scale(d_sq[i:i + 1], mn, eps, inv, out[i:i + 1])
        got = bits32(out)
        want = np.array([np.float32(O.clip_coefficient(x, mn, eps) * inv) for x in sqs],
                        dtype=np.float32).view(np.uint32)
        assert_bits_equal(got, want, f"max_norm {mn}, eps {eps}, inv_loss_scale {inv}")


def test_device_scale_step_equals_host_scale_step():
    """The fused step with its grad scale read from device memory gives the bits of the same step
    with that scale passed from the host: bf16 replicas, a ragged tail, the skip flag off and on."""
    n, R = 9 * TILE + 77, 8
    rng = np.random.default_rng(5)
    reps = [dev_rep(r, "bf16") for r in _reps_np(rng, R, n, "bf16")]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = Z.adam_hparams(lr=1e-3, weight_decay=0.01, step=3)
    for gs in (1.0, 0.37, 2.0 ** -20):
        for skip_val in (0, 1):
            res = []
            for dev_scale in (False, True):
                d_p, d_m, d_v = dev_f32(master), torch.full((n,), 1e-4, device=DEV), torch.full((n,), 1e-8, device=DEV)
                d_o = empty16(n, "bf16", fill=0.0)
                skip = torch.full((1,), skip_val, dtype=torch.int32, device=DEV)
                if dev_scale:
                    d_gs = torch.full((1,), gs, device=DEV)
                    Z.zero_adam_shard_step_dev_scale(reps, n, d_gs, d_p, d_m, d_v, hp, out=d_o, skip=skip)
                else:
                    Z.zero_adam_shard_step(reps, n, gs, d_p, d_m, d_v, hp, out=d_o, skip=skip)
                torch.cuda.synchronize()
                res.append((bits32(d_p), bits32(d_m), bits32(d_v), bits16(d_o)))
            for a, b, what in zip(res[0], res[1], ("master", "m", "v", "params")):
                assert_bits_equal(b, a, f"gs {gs} skip {skip_val} {what}")
            if skip_val:
                assert_bits_equal(res[1][0], f32_bits(master), "skipped master")


def test_device_step_counter_equals_host_steps():
    """zero_adam_shard_step_dev_t over steps t = 3..6 (t, constants and grad scale read on the
    device, t advanced on the device) gives the bits of the same steps with t from the host; a
    skipped step leaves the state and t alone; t = 7, past the 6-entry table, writes nothing, keeps
    t and sets the status word; n = 0 only runs the counter kernel."""
    n, R, t0 = 7 * TILE + 45, 8, 3
    rng = np.random.default_rng(17)
    reps = [dev_rep(r, "bf16") for r in _reps_np(rng, R, n, "bf16")]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    kw = dict(lr=1e-3, weight_decay=0.01, wd_mode="adamw")
    table = Z.adam_table(Z.adam_hparams(**kw), 6, device=DEV)          # steps 1..6
    dev = [dev_f32(master), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)]
    host = [t.clone() for t in dev]
    d_out, h_out = empty16(n, "bf16"), empty16(n, "bf16")
    step = torch.full((1,), t0, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gs = torch.full((1,), 0.75, device=DEV)
    skip = torch.zeros(1, dtype=torch.int32, device=DEV)
    t_host = t0
    for k, skipped in enumerate((False, False, True, False, False, False, False)):
        skip.fill_(1 if skipped else 0)
        Z.zero_adam_shard_step_dev_t(reps, n, gs, table, step, status, *dev, wd_mode="adamw", out=d_out,
                                     skip=skip)
        if t_host <= 6:                # the host steps only where the table has constants
            Z.zero_adam_shard_step(reps, n, 0.75, *host, Z.adam_hparams(step=t_host, **kw),
                                   out=h_out, skip=skip)
        torch.cuda.synchronize()
        refused = t_host > 6 and not skipped
        if not skipped and not refused:
            t_host += 1
        assert int(step.item()) == t_host, k
        assert int(status.item()) == (Z.ZERO_DEV_T_OUT_OF_TABLE if t_host > 6 and refused else 0), k
        for a, b, what in zip(dev, host, ("master", "m", "v")):
            assert_bits_equal(bits32(a), bits32(b), f"step {k} {what}")
        assert_bits_equal(bits16(d_out), bits16(h_out), f"step {k} params")
    assert t_host == 7 and int(status.item()) == Z.ZERO_DEV_T_OUT_OF_TABLE
    status.zero_()
    step.fill_(6)
    before = bits32(dev[0])
    Z.zero_adam_shard_step_dev_t(reps, 0, gs, table, step, status, *dev)
    torch.cuda.synchronize()
    assert int(step.item()) == 7 and int(status.item()) == 0
    assert_bits_equal(bits32(dev[0]), before, "n = 0")


@pytest.mark.parametrize("t", [5, 4, 0, -3, 2 ** 40])
def test_device_step_outside_table_refuses_update(t):
    """A 3-entry constants table driven to a t it has no entry for (past it, at 0 or below, or
    far past): master, m, v and the slot keep their bits, t stays, the status word is set. The
    same call at t = 3 then updates as the host step does."""
    n, R = 5 * TILE + 17, 8
    rng = np.random.default_rng(41)
    reps = [dev_rep(r, "bf16") for r in _reps_np(rng, R, n, "bf16")]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    kw = dict(lr=1e-3, weight_decay=0.01, wd_mode="adamw")
    table = Z.adam_table(Z.adam_hparams(**kw), 3, device=DEV)
    dev = [dev_f32(master), dev_f32(np.full(n, 1e-4, np.float32)), dev_f32(np.full(n, 1e-8, np.float32))]
    before = [bits32(x) for x in dev]
    d_out = empty16(n, "bf16", fill=-5.0)
    out_before = bits16(d_out)
    step = torch.full((1,), t, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gs = torch.ones(1, device=DEV)
    for _ in range(2):                 # twice: still refused, still no advance
        Z.zero_adam_shard_step_dev_t(reps, n, gs, table, step, status, *dev, out=d_out)
    torch.cuda.synchronize()
    assert int(step.item()) == t and int(status.item()) == Z.ZERO_DEV_T_OUT_OF_TABLE
    for a, b, what in zip(dev, before, ("master", "m", "v")):
        assert_bits_equal(bits32(a), b, f"refused {what}")
    assert_bits_equal(bits16(d_out), out_before, "refused slot")
    # back inside the table: the update runs and matches the host step
    step.fill_(3)
    host = [x.clone() for x in dev]
    h_out = empty16(n, "bf16")
    Z.zero_adam_shard_step_dev_t(reps, n, gs, table, step, status, *dev, out=d_out)
    Z.zero_adam_shard_step(reps, n, 1.0, *host, Z.adam_hparams(step=3, **kw), out=h_out)
    torch.cuda.synchronize()
    assert int(step.item()) == 4
    for a, b, what in zip(dev, host, ("master", "m", "v")):
        assert_bits_equal(bits32(a), bits32(b), f"t = 3 {what}")
    assert_bits_equal(bits16(d_out), bits16(h_out), "t = 3 params")


# --- IEEE special cases inside the update: subnormals, overflow, 0/0, inf/inf, signed zeros ----------


@pytest.mark.parametrize("case", range(len(EXTREME_CASES)))
@pytest.mark.parametrize("rep", ["f32", "bf16"])
def test_step_ieee_special_cases(case, rep):
    """Operands drawn over the whole binary32 range, so that subnormal inputs and results, overflow,
    0/0 and inf/inf arise inside the update. Every non-NaN fp32 and 16-bit result equals the oracle's
    bit for bit; NaN results must be NaN on both sides."""
    regimes, gs, hpx = EXTREME_CASES[case]
    n = 5 * TILE + 77
    rng = np.random.default_rng(700 + case)
    g, p, m, v = mixed_state(rng, n, regimes)
    if rep == "f32":
        reps = g[None, :].copy()
    else:   # three bf16 replicas whose exact fp32 sum spans the same range
        third = (g.view(np.uint32) & 0xFFFF0000).view(np.float32)
        reps = np.stack([(third.view(np.uint32) >> 16).astype(np.uint16)] * 3)
    hp_kw = {**HP, **hpx}
    banner(f"ieee special cases {case} {rep} {regimes} gs={gs}")
    for out_dtype in ("bf16", "f16"):
        got = _run_step(reps, rep, n, p, m, v, hp_kw, out_dtype, grad_scale=gs)
        with np.errstate(all="ignore"):
            want = O.sharded_step(list(reps), rep, gs, p, m, v, O.AdamHParams(**hp_kw), out_dtype)
        for k, what in enumerate(("master", "m", "v")):
            assert_bits_equal_nan(got[k], f32_bits(want[k]), f"{what} ({out_dtype})")
        assert_bits_equal_nan(got[3], want[3], f"out {out_dtype}", out_dtype)


@pytest.mark.parametrize("gs", [1.0, 2.0 ** -16])
def test_step_every_fp16_gradient_pattern(gs):
    """One fp16 replica holding every binary16 pattern (subnormals, infinities, NaNs), widened
    exactly and pushed through the update from warm state."""
    h = f16_all_patterns()
    n = h.size
    rng = np.random.default_rng(77)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    banner(f"every fp16 gradient pattern gs={gs}")
    got = _run_step(h[None, :], "f16", n, p, m, v, HP, "bf16", grad_scale=gs)
    with np.errstate(all="ignore"):
        want = O.sharded_step([h], "f16", gs, p, m, v, O.AdamHParams(**HP), "bf16")
    for k, what in enumerate(("master", "m", "v")):
        assert_bits_equal_nan(got[k], f32_bits(want[k]), what)
    assert_bits_equal_nan(got[3], want[3], "out", "bf16")


def test_reduce_and_sqnorm_over_the_full_range():
    """The reduce pass over finite operands spanning every binade: the fp32 sum bit for bit and
    the fp64 squared norm against an exact sum of the same squares."""
    n = 7 * TILE + 301
    rng = np.random.default_rng(91)
    reps = np.stack([f32_patterns(rng, n, "full") * np.float32(2.0 ** -2) for _ in range(3)])
    banner("reduce over the full fp32 range")
    d_r = [dev_f32(r) for r in reps]
    d_g = torch.empty(n, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    Z.zero_reduce_shard(d_r, n, d_g, nonfinite=flag, sq_partials=parts, sq_scale=2.0 ** -16)
    Z.zero_shard_sqnorm(None, n, 2.0 ** -16, parts, sq)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        acc = O.replica_sum(list(reps), "f32")
    assert_bits_equal(bits32(d_g), f32_bits(acc), "reduced gradient")
    assert int(flag.item()) == int(O.nonfinite_flag(acc))
    finite = np.isfinite(acc)
    if finite.all():
        want = O.shard_sqnorm(acc, 2.0 ** -16)
        assert abs(sq.item() - want) <= 1e-10 * want
    else:
        assert math.isinf(sq.item()) or math.isnan(sq.item())


def test_prepared_step_equals_the_plain_call():
    """AdamStep (arrays marshalled once) gives the bits zero_adam_shard_step gives, step after step."""
    n = 5 * TILE + 77
    rng = np.random.default_rng(44)
    reps = _reps_np(rng, 3, n, "bf16")
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    runs = []
    for prepared in (False, True):
        d_r = [dev_rep(r, "bf16") for r in reps]
        d_p, d_m, d_v = dev_f32(master), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
        d_o = empty16(n, "bf16")
        call = Z.AdamStep(d_r, n, d_p, d_m, d_v, out=d_o) if prepared else None
        for t, gs in ((1, 1.0), (2, 0.5)):
            hp = Z.adam_hparams(lr=1e-3, weight_decay=0.01, step=t)
            if prepared:
                call(gs, hp)
            else:
                Z.zero_adam_shard_step(d_r, n, gs, d_p, d_m, d_v, hp, out=d_o)
        torch.cuda.synchronize()
        runs.append((bits32(d_p), bits32(d_m), bits32(d_v), bits16(d_o)))
    for a, b, what in zip(runs[0], runs[1], ("master", "m", "v", "out")):
        assert_bits_equal(b, a, what)


def test_prepared_reduce_equals_the_plain_call():
    """ReduceCall (arrays marshalled once) writes the gradient, flag and partials zero_reduce_shard
    writes, call after call, over several tiles and a ragged tail."""
    n = 6 * TILE + 91
    rng = np.random.default_rng(45)
    reps = _reps_np(rng, 5, n, "f16")
    d_r = [dev_rep(r, "f16") for r in reps]
    runs = []
    for prepared in (False, True):
        g = torch.full((n,), float("nan"), device=DEV)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        parts = torch.full((Z.zero_sq_partials_len(n),), -1.0, dtype=torch.float64, device=DEV)
        call = Z.ReduceCall(d_r, n, g, flag, parts) if prepared else None
        for scale in (2.0 ** -16, 0.5):
            if prepared:
                call(scale)
            else:
                Z.zero_reduce_shard(d_r, n, g, flag, parts, scale)
        torch.cuda.synchronize()
        runs.append((bits32(g), int(flag.item()), parts.cpu().numpy().view(np.uint64).copy()))
    assert_bits_equal(runs[1][0], runs[0][0], "gradient")
    assert runs[1][1] == runs[0][1] == 0
    assert np.array_equal(runs[1][2], runs[0][2])
    assert_bits_equal(runs[1][0], f32_bits(O.replica_sum(list(reps), "f16")), "gradient vs oracle")


def test_concurrent_steps_from_host_threads():
    """Six host threads, each with its own stream and arrays, step at the same time: every result
    equals the oracle's bit for bit (launch setup, the CU-count cache and error state are safe to use
    from several threads)."""
    import threading

    n = 7 * TILE + 333
    jobs = []
    for k in range(6):
        rng = np.random.default_rng(500 + k)
        reps = _reps_np(rng, 1 + k, n, ["bf16", "f16", "f32"][k % 3])
        master = (rng.standard_normal(n) * 0.02).astype(np.float32)
        jobs.append((reps, ["bf16", "f16", "f32"][k % 3], master))
    hp = {k: v for k, v in HP.items() if k != "step"}
    out = [None] * len(jobs)
    barrier = threading.Barrier(len(jobs), timeout=60)

    def work(k):
        reps, dt, master = jobs[k]
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            d_r = [dev_rep(r, dt) for r in reps]
            d_p = dev_f32(master)
            d_m, d_v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
            d_o = empty16(n, "bf16")
            s.synchronize()
            barrier.wait()
            for t in (1, 2, 3):
                Z.zero_adam_shard_step(d_r, n, 1.0, d_p, d_m, d_v, Z.adam_hparams(step=t, **hp), out=d_o)
            s.synchronize()
        out[k] = (bits32(d_p), bits16(d_o))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for k, (reps, dt, master) in enumerate(jobs):
        p, m, v = master, np.zeros(n, np.float32), np.zeros(n, np.float32)
        for t in (1, 2, 3):
            p, m, v, o = O.sharded_step(list(reps), dt, 1.0, p, m, v, O.AdamHParams(step=t, **hp), "bf16")
        assert out[k] is not None, f"thread {k} did not finish"
        assert_bits_equal(out[k][0], f32_bits(p), f"master, thread {k}")
        assert_bits_equal(out[k][1], o, f"out, thread {k}")
