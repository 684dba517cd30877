"""GPU parity on the degenerate and limit cases of the sharded step.

  * resume: k steps in a row equal j steps, a save of the rank's state (master, m, v and the step
    count t) to host memory, a restore into fresh device buffers, and k - j more steps, bit for bit;
  * Nd = 1: the single rank's shard is the whole flat space, so the step equals the oracle's
    unsharded data-parallel Adam;
  * N < Nd: the trailing ranks own padding only, which stays zero;
  * a shard of more than 2^33 elements in one call: element indices past 2^32 and a tile count past
    the per-launch grid limit (2^24 blocks), checked on windows at the head, across the grid
    boundary and at the ragged tail.
"""

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, banner, bits16, bits32, dev_f32, dev_rep, empty16, f32_bits

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _bf16_reps(rng, R, n, std=1e-3):
    x = rng.standard_normal((R, n)).astype(np.float32) * np.float32(std)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_resume_after_save_and_restore_is_bitwise():
    n, R, k, j = 3 * 512 * 7 + 129, 8, 5, 2
    banner(f"resume n={n} k={k} j={j}")
    rng = np.random.default_rng(11)
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [_bf16_reps(rng, R, n) for _ in range(k)]        # a fresh replica set every step

    def run(state, steps):
        p, m, v, out, t = state
        for s in steps:
            Z.zero_adam_shard_step([dev_rep(r, "bf16") for r in grads[s]], n, 1.0, p, m, v,
                                   Z.adam_hparams(step=t, **HP), out=out)
            t += 1
        torch.cuda.synchronize()
        return p, m, v, out, t

    straight = run((dev_f32(master0), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                    empty16(n, "bf16"), 1), range(k))
    part = run((dev_f32(master0), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                empty16(n, "bf16"), 1), range(j))
    saved = {"master": part[0].cpu(), "m": part[1].cpu(), "v": part[2].cpu(), "t": part[4]}
    del part
    restored = (saved["master"].to(DEV), saved["m"].to(DEV), saved["v"].to(DEV), empty16(n, "bf16"),
                saved["t"])
    resumed = run(restored, range(j, k))
    assert resumed[4] == straight[4] == k + 1
    for a, b, what in zip(straight[:3], resumed[:3], ("master", "m", "v")):
        assert_bits_equal(bits32(b), bits32(a), f"resumed {what}")
    assert_bits_equal(bits16(resumed[3]), bits16(straight[3]), "resumed bf16 params")
    # and both equal the oracle's k steps
    p, m, v = master0, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for s in range(k):
        p, m, v, o = O.sharded_step(list(grads[s]), "bf16", 1.0, p, m, v, O.AdamHParams(step=s + 1, **HP), "bf16")
    assert_bits_equal(bits32(straight[0]), f32_bits(p), "master vs oracle")
    assert_bits_equal(bits16(straight[3]), o, "params vs oracle")


def test_single_rank_is_unsharded_adam():
    n = 100_003
    plan = Z.zero_partition_plan(n, 1)
    assert (plan.shard_elems, plan.padded_n, plan.pad) == (n, n, 0)
    assert Z.zero_shard_range(plan, 0) == (0, n)
    rng = np.random.default_rng(12)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    d_p, d_m, d_v = dev_f32(master), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    d_o = empty16(n, "f16")
    for t in (1, 2):
        Z.zero_adam_shard_step([dev_f32(g)], n, 1.0, d_p, d_m, d_v, Z.adam_hparams(step=t, **HP), out=d_o)
    torch.cuda.synchronize()
    p, m, v = master, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in (1, 2):
        p, m, v, o = O.unsharded_step(g, p, m, v, O.AdamHParams(step=t, **HP), out_dtype="f16")
    assert_bits_equal(bits32(d_p), f32_bits(p), "master")
    assert_bits_equal(bits32(d_m), f32_bits(m), "m")
    assert_bits_equal(bits32(d_v), f32_bits(v), "v")
    assert_bits_equal(bits16(d_o), o, "fp16 params")


@pytest.mark.parametrize("n,nd", [(5, 8), (1, 4), (0, 3), (9, 16)])
def test_fewer_elements_than_ranks(n, nd):
    """Every rank steps its slice of shared flat buffers; ranks past N own padding only."""
    plan = Z.zero_partition_plan(n, nd)
    S, P = plan.shard_elems, plan.padded_n
    rng = np.random.default_rng(13)
    master = np.zeros(P, np.float32)
    master[:n] = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grad = np.zeros(P, np.float32)
    grad[:n] = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    d_p, d_m, d_v, d_g = (dev_f32(master), torch.zeros(max(P, 1), device=DEV),
                          torch.zeros(max(P, 1), device=DEV), dev_f32(grad))
    d_o = empty16(max(P, 1), "bf16", fill=3.0)
    for r in range(nd):
        b, valid = Z.zero_shard_range(plan, r)
        assert valid == max(0, min(S, n - b))
        Z.zero_adam_shard_step([d_g[b:b + S]], S, 1.0, d_p[b:b + S], d_m[b:b + S], d_v[b:b + S],
                               Z.adam_hparams(step=1, **HP), out=d_o[b:b + S])
    torch.cuda.synchronize()
    p, m, v, o = O.unsharded_step(grad, master, np.zeros(P, np.float32), np.zeros(P, np.float32),
                                  O.AdamHParams(step=1, **HP), out_dtype="bf16")
    assert_bits_equal(bits32(d_p)[:P], f32_bits(p), "master")
    assert_bits_equal(bits32(d_m)[:P], f32_bits(m), "m")
    assert_bits_equal(bits16(d_o)[:P], o, "gathered params")
    assert not bits32(d_p)[n:P].any() and not bits16(d_o)[n:P].any()      # padding stays 0


def test_shard_past_2_pow_33_elements():
    """One call over n = 2^33 + 5000 elements: 33,554,451 whole 256-element tiles in three grids of
    at most 2^24 blocks, and a 136-element remainder taken by the last grid's extra block. One bf16
    replica, bf16 output: about 137 GB of device memory."""
    n = (1 << 33) + 5000
    tile = 256                                        # Adam kernel tile
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    banner(f"huge shard n={n}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(14)
    rep = (torch.randn(n, generator=gen, device=DEV) * 1e-3).to(torch.bfloat16)
    master = torch.randn(n, generator=gen, device=DEV).mul_(0.02)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    out = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    boundary = (1 << 24) * tile                       # first element of the second grid (2^32)
    wins = [(0, 1 << 16), (boundary - 4099, boundary + 4099), (2 * boundary - 777, 2 * boundary + 777),
            (n - 70_000, n)]
    before = {w: bits32(master[w[0]:w[1]]).view(np.float32) for w in wins}
    Z.zero_adam_shard_step([rep], n, 1.0, master, m, v, Z.adam_hparams(step=1, **HP), out=out)
    torch.cuda.synchronize()
    z = None
    for (a, b) in wins:
        r = bits16(rep[a:b])
        z = np.zeros(b - a, np.float32)
        p2, m2, v2, o2 = O.sharded_step([r], "bf16", 1.0, before[(a, b)], z, z, O.AdamHParams(step=1, **HP), "bf16")
        assert_bits_equal(bits32(master[a:b]), f32_bits(p2), f"master [{a},{b})")
        assert_bits_equal(bits32(m[a:b]), f32_bits(m2), f"m [{a},{b})")
        assert_bits_equal(bits32(v[a:b]), f32_bits(v2), f"v [{a},{b})")
        assert_bits_equal(bits16(out[a:b]), o2, f"params [{a},{b})")
    del rep, master, m, v, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
