"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Inputs are drawn on the device (seeded); windows of them are downloaded before the step, the
step runs on the whole shard, and the same windows of the outputs are compared with the oracle
run on the downloaded inputs: bit for bit for fp32 state and 16-bit parameters. The 7B, 13B and
GPT-3 shards sit in one arena placed by zero_arena_layout, as the benchmark places them; the GPT-2
shard uses separate allocations. For the squared
norm, sampled tiles' fp64 partial sums (one per 256-element tile) are recomputed by the oracle from
downloaded replica tiles, and the total is checked against the partials."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, banner, bits16, bits32, f32_bits
from workloads import WORKLOADS
from workloads import device as D
from workloads import host as H
from workloads.placement import step_arrays

pytestmark = pytest.mark.gpu

WIN = 1 << 22                    # elements per checked window
TILE = 256                       # reduce-kernel tile: one squared-norm partial each


def _hp(w, step):
    return dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                wd_mode=w.wd_mode, step=step)


def _windows(S, extra=()):
    mid = (S // 2) // 4 * 4 + 1          # odd start: windows need not be aligned
    return sorted({(0, min(WIN, S)), (mid, min(S, mid + WIN)), (max(0, S - WIN - 3), S), *extra})


def _rep_bits(t):
    return bits32(t) if t.dtype == torch.float32 else bits16(t)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_windows(w, wins, before, reps_win, d_p, d_m, d_v, d_out, hp, grad_scale, out_dtype,
                   rep_offset=lambda a: a):
    for (a, b) in wins:
        p0, m0, v0 = before[(a, b)]
        ra = rep_offset(a)
        reps = reps_win(ra, ra + (b - a))
        p2, m2, v2, o2 = O.sharded_step(list(reps), w.rep_dtype, grad_scale, p0, m0, v0,
                                        O.AdamHParams(**hp), out_dtype)
        assert_bits_equal(bits32(d_p[a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(d_m[a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(d_v[a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(d_out[a:b]), o2, f"params [{a},{b})")


def _placed(w, plan, begin, valid, two_pass=False):
    """The rank's inputs drawn into one arena laid out as the benchmark lays it out."""
    S = plan.shard_elems
    storage, views = Z.arena(step_arrays(w, S, begin, plan.padded_n, two_pass), device=DEV)
    inp = D.rank_inputs(w, begin, S, valid, device=DEV, rep_size=w.window,
                        empty=lambda nm, n, dt: views[nm])
    return storage, views, inp


def _rows(reps, a, b):
    """[R, b - a] copy of elements [a, b) of every replica row (a list of rows or one 2-D tensor)."""
    return torch.stack([r[a:b] for r in reps])


def _bits_to_np(t, dtype):
    if dtype == "f32":
        return bits32(t).view(np.float32)
    return bits16(t)


def test_gpt2_rank3_full_shard():
    """GPT-2 small (124M) over 8 ranks, rank 3: 8 bf16 replicas, AdamW, two steps, whole shard."""
    w = WORKLOADS["gpt2"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S = plan.shard_elems
    banner(f"gpt2 rank {r}: S={S}")
    inp = H.rank_inputs(w, begin, S, valid)
    d_reps = torch.from_numpy(inp["reps"].view(np.int16)).to(DEV).view(torch.bfloat16)
    d_p = torch.from_numpy(inp["master"]).to(DEV)
    d_m = torch.from_numpy(inp["m"]).to(DEV)
    d_v = torch.from_numpy(inp["v"]).to(DEV)
    d_full = torch.zeros(plan.padded_n, dtype=torch.bfloat16, device=DEV)
    p, m, v = inp["master"], inp["m"], inp["v"]
    for t in range(1, w.steps + 1):
        hp = _hp(w, t)
        Z.zero_adam_shard_step(d_reps, S, 1.0, d_p, d_m, d_v, Z.adam_hparams(**hp),
                               out=d_full[begin:begin + S])
        p, m, v, o = O.sharded_step(list(inp["reps"]), "bf16", 1.0, p, m, v, O.AdamHParams(**hp), "bf16")
        torch.cuda.synchronize()
        assert_bits_equal(bits32(d_p), f32_bits(p), f"master step {t}")
        assert_bits_equal(bits32(d_m), f32_bits(m), f"m step {t}")
        assert_bits_equal(bits32(d_v), f32_bits(v), f"v step {t}")
        full = bits16(d_full)
        assert_bits_equal(full[begin:begin + S], o, f"slot step {t}")
        assert not full[:begin].any() and not full[begin + S:].any()


def test_llama7b_shard_full_size():
    """Llama-7B over 8 ranks: one ~842M-element shard, 8 bf16 replicas, warm state at t = 11,
    AdamW; head / middle / tail windows checked bit for bit."""
    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S = plan.shard_elems
    banner(f"llama7b rank {r}: S={S}")
    storage, views, inp = _placed(w, plan, begin, valid)
    d_full = views["full"].zero_()
    wins = _windows(S)
    before = {ab: tuple(bits32(inp[k][ab[0]:ab[1]]).view(np.float32) for k in ("master", "m", "v"))
              for ab in wins}
    hp = _hp(w, w.warm_steps + 1)
    Z.zero_adam_shard_step(inp["reps"], S, 1.0, inp["master"], inp["m"], inp["v"],
                           Z.adam_hparams(**hp), out=d_full[begin:begin + S])
    torch.cuda.synchronize()
    reps_win = lambda a, b: _bits_to_np(_rows(inp["reps"], a, b), "bf16")
    _check_windows(w, wins, before, reps_win, inp["master"], inp["m"], inp["v"],
                   d_full[begin:begin + S], hp, 1.0, "bf16")
    assert torch.isfinite(inp["master"]).all()
    del inp, d_full, views, storage
    _free()


@pytest.mark.parametrize("inject", [False, True])
def test_llama13b_two_pass_full_size(inject):
    """Llama-13B over 16 ranks: 16 fp16 replicas holding grad * 2^16 (with 0.01% +inf injected in
    the second case), reduce -> squared norm -> clip scale -> AdamW with the skip flag, enqueued
    as the benchmark runs it: the clip scale formed on the device, nothing read back before the
    update."""
    w = WORKLOADS["llama13b"]
    if not inject:
        w = dataclasses.replace(w, inf_rate=0.0)
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S = plan.shard_elems
    banner(f"llama13b rank {r}: S={S} inject={inject}")
    storage, views, inp = _placed(w, plan, begin, valid, two_pass=True)
    d_slot = views["slot"].zero_()
    d_g = views["g"]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = torch.empty(Z.zero_sq_partials_len(S), dtype=torch.float64, device=DEV)
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    wins = _windows(S)
    before = {ab: tuple(bits32(inp[k][ab[0]:ab[1]]).view(np.float32) for k in ("master", "m", "v"))
              for ab in wins}
    inv_ls = 1.0 / w.loss_scale
    d_gs = torch.full((1,), float("nan"), device=DEV)
    Z.zero_reduce_shard(inp["reps"], S, d_g, flag, parts, inv_ls)
    Z.zero_shard_sqnorm(None, S, inv_ls, parts, sq)
    Z.zero_clip_scale(sq, w.max_norm, 1e-6, inv_ls, d_gs)
    Z.zero_adam_shard_step_dev_scale([d_g], S, d_gs, inp["master"], inp["m"], inp["v"],
                                     Z.adam_hparams(**_hp(w, 1)), out=d_slot, skip=flag)
    torch.cuda.synchronize()
    flag_h, sq_h, gs = int(flag.item()), float(sq.item()), float(d_gs.item())
    parts_h = parts.cpu().numpy()
    if flag_h == 0:                  # the device's scale is the oracle's formula on the device's norm
        assert np.float32(gs) == np.float32(O.clip_coefficient(sq_h, w.max_norm) * inv_ls)

    # the reduced gradient and the flag, on windows
    any_bad = False
    for (a, b) in wins:
        reps = _bits_to_np(_rows(inp["reps"], a, b), "f16")
        acc = O.replica_sum(list(reps), "f16")
        assert_bits_equal(bits32(d_g[a:b]), f32_bits(acc), f"reduced grad [{a},{b})")
        any_bad |= O.nonfinite_flag(acc)
    assert flag_h == (1 if inject else 0)
    if not inject:
        assert not any_bad
    # squared norm: sampled tiles' partials recomputed from their own replica elements, and the total
    ntiles = math.ceil(S / TILE)
    for t in (0, 1, ntiles // 2, ntiles - 1):
        acc = O.replica_sum(list(_bits_to_np(
            _rows(inp["reps"], t * TILE, min(S, (t + 1) * TILE)), "f16")), "f16")
        want = O.shard_sqnorm(acc, inv_ls)
        if np.isfinite(want):
            assert parts_h[t] == pytest.approx(want, rel=1e-12, abs=0), t
        else:
            assert not np.isfinite(parts_h[t])
    if not inject:
        assert sq_h == pytest.approx(math.fsum(parts_h[:ntiles].tolist()), rel=1e-12, abs=0)
        assert 0.0 < O.clip_coefficient(sq_h, w.max_norm) < 1.0      # clipping is active
    # the update (or its absence), on windows
    for (a, b) in wins:
        p0, m0, v0 = before[(a, b)]
        if inject:
            assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p0), "skipped master")
            assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m0), "skipped m")
            assert not d_slot[a:b].any()
            continue
        reps = _bits_to_np(_rows(inp["reps"], a, b), "f16")
        acc = O.replica_sum(list(reps), "f16")
        p2, m2, v2, o2 = O.sharded_step([acc], "f32", gs, p0, m0, v0, O.AdamHParams(**_hp(w, 1)), "f16")
        assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(inp["v"][a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(d_slot[a:b]), o2, f"fp16 params [{a},{b})")
    del inp, d_g, d_slot, views, storage
    _free()


def test_gpt3_windowed_shard_full_size():
    """GPT-3 175B over 64 ranks: a ~2.73B-element shard stepped in 64 Mi windows (40 full and a
    tail), each window summing the same 64 bf16 replica windows; slot-only output."""
    w = WORKLOADS["gpt3"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S, W = plan.shard_elems, w.window
    banner(f"gpt3 rank {r}: S={S} window={W}")
    storage, views, inp = _placed(w, plan, begin, valid)
    d_slot = views["slot"].zero_()
    last = (S // W) * W
    wins = [(0, WIN), (17 * W + 5, 17 * W + 5 + WIN), (last + 11, last + 11 + WIN), (S - WIN, S)]
    before = {ab: tuple(bits32(inp[k][ab[0]:ab[1]]).view(np.float32) for k in ("master", "m", "v"))
              for ab in wins}
    hp = _hp(w, 1)
    h = Z.adam_hparams(**hp)
    for a in range(0, S, W):
        b = min(S, a + W)
        Z.zero_adam_shard_step(inp["reps"], b - a, 1.0, inp["master"][a:], inp["m"][a:], inp["v"][a:],
                               h, out=d_slot[a:])
    torch.cuda.synchronize()
    reps_win = lambda a, b: _bits_to_np(_rows(inp["reps"], a, b), "bf16")
    _check_windows(w, wins, before, reps_win, inp["master"], inp["m"], inp["v"], d_slot, hp, 1.0,
                   "bf16", rep_offset=lambda a: a % W)
    del inp, d_slot, views, storage
    _free()
