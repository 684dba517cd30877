"""GPU + host parity of the offloaded step (ZeRO-Offload): device replica sum per chunk, copy to
pinned host memory (or the reduce kernel writing there itself, with no device staging), host Adam
on host state, 16-bit parameters copied into the device slot. Bit for bit against the oracle and
against the all-device step on the same inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, banner, bits16, bits32, dev_rep, f32_bits

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _inputs(rng, n, R):
    x = rng.standard_normal((R, n)).astype(np.float32) * np.float32(1e-3)
    reps = (x.view(np.uint32) >> 16).astype(np.uint16)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    return reps, master, m, v


@pytest.mark.parametrize("n,chunk,side,direct", [
    (5 * 4096 + 777, 4096, False, False), (5 * 4096 + 777, 4096, True, False),
    (1000, 4096, False, False), (1, 1, True, False), (3 * 65536, 65536, True, False),
    (64 << 20, 8 << 20, True, False),
    (5 * 4096 + 777, 4096, False, True), (1, 1, True, True), (64 << 20, 8 << 20, True, True)])
def test_offload_step_matches_oracle_and_device_step(n, chunk, side, direct):
    banner(f"offload n={n} chunk={chunk} side={side} direct={direct}")
    rng = np.random.default_rng(n % 997 + chunk)
    R = 8
    reps, master, m, v = _inputs(rng, n, R)
    d_reps = dev_rep(reps.reshape(-1), "bf16").view(R, n)
    hp = Z.adam_hparams(step=4, **HP)
    # offloaded: host state, device slot
    hm, hmm, hv = master.copy(), m.copy(), v.copy()
    slot = torch.full((n + 8,), -1.0, dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream() if side else None
    bufs = Z.offload_buffers(chunk, threads=8, h2d_stream=stream, direct=direct)
    assert (bufs["d_grad"] is None) == direct
    Z.zero_offload_step(d_reps, n, 0.5, hm, hmm, hv, hp, slot[4:4 + n], bufs)
    torch.cuda.synchronize()
    got_slot = bits16(slot)
    assert (got_slot[:4] == got_slot[0]).all() and (got_slot[4 + n:] == got_slot[0]).all()
    # oracle
    p2, m2, v2, o2 = O.sharded_step(list(reps), "bf16", 0.5, master, m, v, O.AdamHParams(step=4, **HP), "bf16")
    assert_bits_equal(hm.view(np.uint32), f32_bits(p2), "host master")
    assert_bits_equal(hmm.view(np.uint32), f32_bits(m2), "host m")
    assert_bits_equal(hv.view(np.uint32), f32_bits(v2), "host v")
    assert_bits_equal(got_slot[4:4 + n], o2, "slot")
    # the all-device step on the same inputs gives the same bits
    dp, dm, dv = (torch.from_numpy(a.copy()).to(DEV) for a in (master, m, v))
    dslot = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    Z.zero_adam_shard_step(d_reps, n, 0.5, dp, dm, dv, hp, out=dslot)
    torch.cuda.synchronize()
    assert_bits_equal(bits32(dp), hm.view(np.uint32), "device vs host master")
    assert_bits_equal(bits16(dslot), got_slot[4:4 + n], "device vs host slot")


def test_offload_fp16_slot_and_l2_mode():
    rng = np.random.default_rng(3)
    n, R = 3 * 5000 + 3, 3
    x = rng.standard_normal((R, n)).astype(np.float32) * np.float32(1e-3 * 1024)
    reps = x.astype(np.float16).view(np.uint16)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z = np.zeros(n, np.float32)
    kw = {**HP, "wd_mode": "l2", "weight_decay": 0.1, "step": 1}
    hm, hmm, hv = master.copy(), z.copy(), z.copy()
    slot = torch.zeros(n, dtype=torch.float16, device=DEV)
    Z.zero_offload_step([dev_rep(r, "f16") for r in reps], n, 1.0 / 1024, hm, hmm, hv, Z.adam_hparams(**kw),
                        slot, Z.offload_buffers(5000, threads=3))
    torch.cuda.synchronize()
    p2, m2, v2, o2 = O.sharded_step(list(reps), "f16", 1.0 / 1024, master, z, z, O.AdamHParams(**kw), "f16")
    assert_bits_equal(hm.view(np.uint32), f32_bits(p2), "host master")
    assert_bits_equal(bits16(slot), o2, "fp16 slot")


def test_offload_rejects_bad_buffers():
    n = 100
    d_rep = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    h = [np.zeros(n, np.float32) for _ in range(3)]
    slot = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    bufs = Z.offload_buffers(64)
    bufs["chunk_elems"] = 0
    with pytest.raises((Z.ZeroError, ValueError)):
        Z.zero_offload_step([d_rep], n, 1.0, *h, Z.adam_hparams(), slot, bufs)
    with pytest.raises(Z.ZeroError):                  # host state aliasing
        Z.zero_offload_step([d_rep], n, 1.0, h[0], h[0], h[2], Z.adam_hparams(), slot, Z.offload_buffers(64))


@pytest.mark.parametrize("seed", range(12))
def test_offload_random_configurations(seed):
    """Seeded random sizes, chunk sizes (also larger than the shard), host thread counts, replica
    counts and dtypes, output dtypes, decay modes, copy-back streams and staging (device buffer
    and copy, or the kernel writing host memory), against the oracle."""
    rng = np.random.default_rng(40_000 + seed)
    n = int(rng.choice([rng.integers(1, 2000), rng.integers(2000, 300_000)]))
    chunk = int(rng.choice([1, 7, 256, 4096, 65536, 1 << 20]))
    threads = int(rng.choice([0, 1, 3, 8]))
    R = int(rng.choice([1, 2, 5, 8, 16]))
    rdt = str(rng.choice(["f32", "f16", "bf16"]))
    odt = str(rng.choice(["bf16", "f16"]))
    mode = str(rng.choice(["adamw", "l2"]))
    side = bool(rng.integers(0, 2))
    banner(f"offload random seed={seed} n={n} chunk={chunk} threads={threads} R={R} {rdt}->{odt} {mode}")
    x = rng.standard_normal((R, n)).astype(np.float32) * np.float32(1e-3)
    if rdt == "f32":
        reps = x
    elif rdt == "bf16":
        reps = (x.view(np.uint32) >> 16).astype(np.uint16)
    else:
        reps = (x * np.float32(64)).astype(np.float16).view(np.uint16)
    d_reps = [dev_rep(r, rdt) for r in reps]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    kw = {**HP, "wd_mode": mode, "step": int(rng.integers(1, 100))}
    direct = bool(rng.integers(0, 2))
    banner(f"  staging: {'kernel writes host memory' if direct else 'device buffer + copy'}")
    hm, hmm, hv = master.copy(), m.copy(), v.copy()
    t16 = torch.bfloat16 if odt == "bf16" else torch.float16
    slot = torch.full((n + 6,), -1.0, dtype=t16, device=DEV)
    bufs = Z.offload_buffers(chunk, threads=threads, h2d_stream=torch.cuda.Stream() if side else None,
                             direct=direct)
    Z.zero_offload_step(d_reps, n, 0.25, hm, hmm, hv, Z.adam_hparams(**kw), slot[3:3 + n], bufs)
    torch.cuda.synchronize()
    p2, m2, v2, o2 = O.sharded_step(list(reps), rdt, 0.25, master, m, v, O.AdamHParams(**kw), odt)
    assert_bits_equal(hm.view(np.uint32), f32_bits(p2), "host master")
    assert_bits_equal(hmm.view(np.uint32), f32_bits(m2), "host m")
    assert_bits_equal(hv.view(np.uint32), f32_bits(v2), "host v")
    got = bits16(slot)
    assert (got[:3] == got[0]).all() and (got[3 + n:] == got[0]).all(), "write outside the slot"
    assert_bits_equal(got[3:3 + n], o2, "slot")


def test_reduce_into_pinned_host_memory():
    """The reduce pass writing straight into pinned host memory (the offloaded step's direct
    staging) gives the bits it gives into device memory, over several tiles and a ragged tail;
    a plain (pageable) host tensor is refused by the binding."""
    rng = np.random.default_rng(77)
    n, R = 3 * 4096 + 123, 5
    reps, _, _, _ = _inputs(rng, n, R)
    d_reps = [dev_rep(r, "bf16") for r in reps]
    h = torch.full((n,), float("nan"), dtype=torch.float32, pin_memory=True)
    d = torch.empty(n, dtype=torch.float32, device=DEV)
    Z.zero_reduce_shard(d_reps, n, h)
    Z.zero_reduce_shard(d_reps, n, d)
    torch.cuda.synchronize()
    assert_bits_equal(h.numpy().view(np.uint32), bits32(d), "pinned vs device")
    assert_bits_equal(h.numpy().view(np.uint32), f32_bits(O.replica_sum(list(reps), "bf16")), "pinned vs oracle")
    with pytest.raises(TypeError):
        Z.zero_reduce_shard(d_reps, n, torch.empty(n, dtype=torch.float32))


def test_offload_direct_staging_refuses_pageable_host_memory():
    """With no device staging the kernel would write h_grad itself, so pageable host memory there
    is refused before anything is enqueued (the state and the slot are left as they were); pinned
    memory of the same size is taken."""
    n = 1000
    rng = np.random.default_rng(8)
    reps, master, m, v = _inputs(rng, n, 2)
    d_reps = [dev_rep(r, "bf16") for r in reps]
    hm, hmm, hv = master.copy(), m.copy(), v.copy()
    slot = torch.full((n,), 7.0, dtype=torch.bfloat16, device=DEV)
    bufs = Z.offload_buffers(256, threads=2, direct=True)
    bufs["h_grad"] = torch.empty(2 * 256, dtype=torch.float32)           # pageable
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_offload_step(d_reps, n, 1.0, hm, hmm, hv, Z.adam_hparams(**HP), slot, bufs)
    assert e.value.status == Z.ZERO_E_INVAL and "pinned host memory" in str(e.value)
    torch.cuda.synchronize()
    assert np.array_equal(hm, master) and np.array_equal(hmm, m) and np.array_equal(hv, v)
    assert (slot == 7.0).all()
    bufs["h_grad"] = torch.empty(2 * 256, dtype=torch.float32, pin_memory=True)
    Z.zero_offload_step(d_reps, n, 1.0, hm, hmm, hv, Z.adam_hparams(**HP), slot, bufs)
    torch.cuda.synchronize()
    p2, _, _, o2 = O.sharded_step(list(reps), "bf16", 1.0, master, m, v, O.AdamHParams(**HP), "bf16")
    assert_bits_equal(hm.view(np.uint32), f32_bits(p2), "host master")
    assert_bits_equal(bits16(slot), o2, "slot")
