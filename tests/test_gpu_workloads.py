"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Inputs are drawn on the device (seeded) and the pre-step state is kept as a device copy; the step
runs on the whole shard, then every element is streamed through the oracle in 16 Mi chunks on host
threads (the inputs downloaded, the oracle run on them, the device's results compared): bit for
bit for the reduced gradient, the fp32 state and the 16-bit parameters, over 100% of each shard.
The squared norm is checked against the oracle's over the whole shard to 1e-10. The 7B, 13B and
GPT-3 shards sit in one arena placed by zero_arena_layout, as the benchmark places them; the GPT-2
shard uses separate allocations."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
import fullshard as FS
from gpu_util import DEV, assert_bits_equal, banner, bits16, bits32, f32_bits
from workloads import WORKLOADS
from workloads import device as D
from workloads import host as H
from workloads.placement import step_arrays

pytestmark = pytest.mark.gpu


def _hp(w, step):
    return dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                wd_mode=w.wd_mode, step=step)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


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


def _whole_fused_check(w, inp, pre, slot, hp, S):
    """Every element of a fused-step shard against the oracle, chunk by chunk: (covered, seconds)."""
    ohp = O.AdamHParams(**hp)

    def work(a, b):
        reps = _bits_to_np(_rows(inp["reps"], a, b), w.rep_dtype)
        p0, m0, v0 = (bits32(pre[k][a:b]).view(np.float32) for k in ("master", "m", "v"))
        p2, m2, v2, o2 = O.sharded_step(list(reps), w.rep_dtype, 1.0, p0, m0, v0, ohp, w.out_dtypes[0])
        assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(inp["v"][a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(slot[a:b]), o2, f"params [{a},{b})")

    return FS.run_chunks(S, work)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("slot_off", [0, 1])
def test_llama7b_shard_full_size(slot_off):
    """Llama-7B over 8 ranks: one ~842M-element shard, 8 bf16 replicas, warm state at t = 11,
    AdamW; every element of master, m, v and the slot checked bit for bit. With slot_off = 1 the
    slot starts one element past its place in the gathered buffer (2 bytes past a 4-byte word, as
    rank r's slot r*S is when S is odd), which takes the word-realigning store path; the elements
    just outside the slot must keep their canary."""
    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S = plan.shard_elems
    banner(f"llama7b rank {r}: S={S} slot offset {slot_off}")
    specs = [(nm, n + (slot_off if nm == "full" else 0), dt, g, h)
             for nm, n, dt, g, h in step_arrays(w, S, begin, plan.padded_n)]
    storage, views = Z.arena(specs, device=DEV)
    inp = D.rank_inputs(w, begin, S, valid, device=DEV, rep_size=w.window,
                        empty=lambda nm, n, dt: views[nm])
    d_full = views["full"].fill_(-3.0)
    slot = d_full[begin + slot_off:begin + slot_off + S]
    pre = {k: inp[k].clone() for k in ("master", "m", "v")}
    hp = _hp(w, w.warm_steps + 1)
    Z.zero_adam_shard_step(inp["reps"], S, 1.0, inp["master"], inp["m"], inp["v"],
                           Z.adam_hparams(**hp), out=slot)
    torch.cuda.synchronize()
    covered, secs = _whole_fused_check(w, inp, pre, slot, hp, S)
    banner(f"llama7b slot offset {slot_off}: {covered} of {S} elements ({100.0 * covered / S:.1f}%) "
           f"bit-exact in {secs:.1f} s")
    assert covered == S
    canary = torch.full((1,), -3.0, dtype=torch.bfloat16, device=DEV)
    assert bool((d_full[:begin + slot_off] == canary).all()) and bool((d_full[begin + slot_off + S:] == canary).all())
    assert torch.isfinite(inp["master"]).all()
    del inp, pre, d_full, slot, views, storage
    _free()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("direct", [False, True])
def test_llama7b_offloaded_step_full_size(direct):
    """The 7B shard's step offloaded as the benchmark runs it (ZeRO-Offload): master, m and v in
    host memory, 32 Mi-element chunks, 16 host threads, the gradient chunks copied from device
    staging or (direct) written into pinned host memory by the reduce kernel. Every element of the
    host state and of the device slot checked bit for bit against the oracle; the elements just
    outside the slot keep their canary."""
    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S = plan.shard_elems
    banner(f"llama7b offloaded rank {r}: S={S} direct={direct}")
    inp = D.rank_inputs(w, begin, S, valid, device=DEV)
    host = {k: inp[k].cpu().numpy() for k in ("master", "m", "v")}
    pre = {k: a.copy() for k, a in host.items()}
    del inp["master"], inp["m"], inp["v"]
    _free()
    d_out = torch.full((S + 2,), -3.0, dtype=torch.bfloat16, device=DEV)
    slot = d_out[1:1 + S]
    hp = _hp(w, w.warm_steps + 1)
    Z.zero_offload_step(inp["reps"], S, 1.0, host["master"], host["m"], host["v"], Z.adam_hparams(**hp),
                        slot, Z.offload_buffers(32 << 20, threads=16, direct=direct))
    torch.cuda.synchronize()
    ohp = O.AdamHParams(**hp)

    def work(a, b):
        reps = _bits_to_np(_rows(inp["reps"], a, b), w.rep_dtype)
        p2, m2, v2, o2 = O.sharded_step(list(reps), w.rep_dtype, 1.0, pre["master"][a:b], pre["m"][a:b],
                                        pre["v"][a:b], ohp, w.out_dtypes[0])
        assert_bits_equal(host["master"][a:b].view(np.uint32), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(host["m"][a:b].view(np.uint32), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(host["v"][a:b].view(np.uint32), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(slot[a:b]), o2, f"params [{a},{b})")

    covered, secs = FS.run_chunks(S, work)
    banner(f"llama7b offloaded (direct={direct}): {covered} of {S} elements "
           f"({100.0 * covered / S:.1f}%) bit-exact in {secs:.1f} s")
    assert covered == S
    ends = bits16(d_out[0:1]).tolist() + bits16(d_out[S + 1:S + 2]).tolist()
    assert ends == [int(O.cast_bf16_rne(np.float32([-3.0]))[0])] * 2
    del inp, host, pre, d_out, slot
    _free()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("inject", [False, True])
def test_llama13b_two_pass_full_size(inject):
    """Llama-13B over 16 ranks: 16 fp16 replicas holding grad * 2^16 (with 0.01% +inf injected in
    the second case), reduce -> squared norm -> clip scale -> AdamW with the skip flag, enqueued
    as the benchmark runs it: the clip scale formed on the device, nothing read back before the
    update. Every element of the reduced gradient and of the update (or of the state left alone
    on the skip) is checked bit for bit; the squared norm against the oracle's over the whole
    shard to 1e-10."""
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
    pre = {k: inp[k].clone() for k in ("master", "m", "v")}
    inv_ls = 1.0 / w.loss_scale
    d_gs = torch.full((1,), float("nan"), device=DEV)
    Z.zero_reduce_shard(inp["reps"], S, d_g, flag, parts, inv_ls)
    Z.zero_shard_sqnorm(None, S, inv_ls, parts, sq)
    Z.zero_clip_scale(sq, w.max_norm, 1e-6, inv_ls, d_gs)
    Z.zero_adam_shard_step_dev_scale([d_g], S, d_gs, inp["master"], inp["m"], inp["v"],
                                     Z.adam_hparams(**_hp(w, 1)), out=d_slot, skip=flag)
    torch.cuda.synchronize()
    flag_h, sq_h, gs = int(flag.item()), float(sq.item()), float(d_gs.item())

    # pass 1: the reduced gradient of every element, and the oracle's sum kept for the norm
    acc_full = np.empty(S, np.float32)
    bad = []

    def reduce_work(a, b):
        acc = O.replica_sum(list(_bits_to_np(_rows(inp["reps"], a, b), "f16")), "f16")
        acc_full[a:b] = acc
        assert_bits_equal(bits32(d_g[a:b]), f32_bits(acc), f"reduced grad [{a},{b})")
        if O.nonfinite_flag(acc):
            bad.append(a)

    covered, secs = FS.run_chunks(S, reduce_work)
    banner(f"llama13b reduce: {covered} of {S} elements ({100.0 * covered / S:.1f}%) bit-exact in "
           f"{secs:.1f} s")
    assert covered == S
    assert flag_h == (1 if bad else 0) == (1 if inject else 0)
    want_sq = O.shard_sqnorm(acc_full, inv_ls)
    if inject:
        assert not math.isfinite(want_sq) and not math.isfinite(sq_h)
    else:
        assert abs(sq_h - want_sq) <= 1e-10 * want_sq, (sq_h, want_sq)
        assert 0.0 < O.clip_coefficient(sq_h, w.max_norm) < 1.0      # clipping is active
        # the device's scale is the oracle's formula on the device's norm
        assert np.float32(gs) == np.float32(O.clip_coefficient(sq_h, w.max_norm) * inv_ls)

    # pass 2: the update of every element (or the state left alone)
    ohp = O.AdamHParams(**_hp(w, 1))

    def update_work(a, b):
        p0, m0, v0 = (bits32(pre[k][a:b]).view(np.float32) for k in ("master", "m", "v"))
        if inject:
            assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p0), f"skipped master [{a},{b})")
            assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m0), f"skipped m [{a},{b})")
            assert_bits_equal(bits32(inp["v"][a:b]), f32_bits(v0), f"skipped v [{a},{b})")
            assert not bits16(d_slot[a:b]).any(), f"skipped slot [{a},{b})"
            return
        p2, m2, v2, o2 = O.sharded_step([acc_full[a:b]], "f32", gs, p0, m0, v0, ohp, "f16")
        assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(inp["v"][a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(d_slot[a:b]), o2, f"fp16 params [{a},{b})")

    covered, secs = FS.run_chunks(S, update_work)
    banner(f"llama13b update: {covered} of {S} elements ({100.0 * covered / S:.1f}%) bit-exact in "
           f"{secs:.1f} s")
    assert covered == S
    del inp, pre, d_g, d_slot, views, storage
    _free()


@pytest.mark.timeout(900)
def test_gpt3_windowed_shard_full_size():
    """GPT-3 175B over 64 ranks: a ~2.73B-element shard stepped in 64 Mi windows (40 full and a
    tail), each window summing the same 64 bf16 replica windows; slot-only output. The oracle's
    replica sum of the window is formed once (every window reads the same replicas), and every
    element of the shard's update is checked bit for bit."""
    w = WORKLOADS["gpt3"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    r = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, r)
    S, W = plan.shard_elems, w.window
    banner(f"gpt3 rank {r}: S={S} window={W}")
    storage, views, inp = _placed(w, plan, begin, valid)
    d_slot = views["slot"].zero_()
    pre = {k: inp[k].clone() for k in ("master", "m", "v")}
    hp = _hp(w, 1)
    h = Z.adam_hparams(**hp)
    for a in range(0, S, W):
        b = min(S, a + W)
        Z.zero_adam_shard_step(inp["reps"], b - a, 1.0, inp["master"][a:], inp["m"][a:], inp["v"][a:],
                               h, out=d_slot[a:])
    torch.cuda.synchronize()
    acc_win = np.empty(W, np.float32)

    def window_sum(a, b):
        acc_win[a:b] = O.replica_sum(list(_bits_to_np(_rows(inp["reps"], a, b), "bf16")), "bf16")

    covered, secs = FS.run_chunks(W, window_sum)
    assert covered == W
    banner(f"gpt3: oracle replica sum of the window in {secs:.1f} s")
    ohp = O.AdamHParams(**hp)
    assert W % FS.CHUNK == 0               # a chunk never straddles two windows

    def work(a, b):
        p0, m0, v0 = (bits32(pre[k][a:b]).view(np.float32) for k in ("master", "m", "v"))
        acc = acc_win[a % W:a % W + (b - a)]
        p2, m2, v2, o2 = O.sharded_step([acc], "f32", 1.0, p0, m0, v0, ohp, "bf16")
        assert_bits_equal(bits32(inp["master"][a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(inp["m"][a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(inp["v"][a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(d_slot[a:b]), o2, f"params [{a},{b})")

    covered, secs = FS.run_chunks(S, work)
    banner(f"gpt3: {covered} of {S} elements ({100.0 * covered / S:.1f}%) bit-exact in {secs:.1f} s")
    assert covered == S
    del inp, pre, d_slot, views, storage
    _free()
