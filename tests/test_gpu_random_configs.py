"""Seeded random configurations of the fused step, the reduce pass and the ZeRO-3 gather against
the oracle, beyond the parametrized grids.

Step and reduce cases draw sizes up to 5000 (ragged against every tile), 1..64 replicas of any
dtype, either output dtype or none, both decay modes, a random grad scale and step, per-array
element offsets (so the vector path, the per-element path and the partial last tile all occur) and
the skip flag; odd seeds pass the grad scale in device memory (zero_adam_shard_step_dev_scale),
and every fourth seed also the step, with constants tables of 1, 7 or 2500 entries
(zero_adam_shard_step_dev_t: a step past its table must write nothing and set the status word).
Odd element offsets put 16-bit arrays 2 bytes past a 4-byte word, and any offset puts fp32 arrays
off 16 bytes, so the word-realigning vector path is drawn often.
Gather cases draw shard counts and sizes, ranges, element sizes and source and
output offsets. Every fp32 and 16-bit result is compared bit for bit, the squared norm to 1e-10.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, banner, bits16, bits32, dev_f32, dev_rep, f32_bits

pytestmark = pytest.mark.gpu

CASES = 300
_T16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def _draw_reps(rng, R, n, dtype):
    x = (rng.standard_normal((R, n)) * rng.choice([1e-4, 1e-3, 1e-1])).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return (x * np.float32(256.0)).astype(np.float16).view(np.uint16)


def _placed(a, off, dtype):
    """Device copy of ``a`` starting ``off`` elements into its own allocation."""
    pad = np.zeros(off, a.dtype)
    if dtype == "f32":
        return dev_f32(np.concatenate([pad, a]))[off:]
    return dev_rep(np.concatenate([pad, a]), dtype)[off:]


def _config(rng):
    return dict(
        n=int(rng.choice([rng.integers(1, 300), rng.integers(300, 5001)])),
        R=int(rng.choice([1, 2, 3, 7, 8, 9, 16, 17, 33, 64])),
        rdt=str(rng.choice(["f32", "f16", "bf16"])),
        odt=[None, "bf16", "f16"][int(rng.integers(0, 3))],
        mode=str(rng.choice(["adamw", "l2"])),
        gs=float(np.float32(rng.choice([1.0, 0.5, 2.0 ** -8, float(rng.uniform(0.01, 3))]))),
        step=int(rng.integers(1, 2000)),
        wd=float(rng.choice([0.0, 0.01, 0.1])),
        offs=[int(x) if rng.random() < 0.5 else 0 for x in rng.integers(0, 8, 5)],
        skip=[None, 0, 1][int(rng.integers(0, 3))],
    )


@pytest.mark.parametrize("seed", range(CASES))
def test_random_fused_step(seed):
    rng = np.random.default_rng(10_000 + seed)
    c = _config(rng)
    n, R = c["n"], c["R"]
    banner(f"random fused step seed={seed} {c}")
    reps = _draw_reps(rng, R, n, c["rdt"])
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    o_rep, o_p, o_m, o_v, o_out = c["offs"]
    d_reps = [_placed(r, o_rep, c["rdt"]) for r in reps]
    d_p, d_m, d_v = _placed(p, o_p, "f32"), _placed(m, o_m, "f32"), _placed(v, o_v, "f32")
    d_out = None
    if c["odt"]:
        full = torch.full((n + o_out + 3,), -2.0, dtype=_T16[c["odt"]], device=DEV)
        d_out = full[o_out:o_out + n]
    skip = None if c["skip"] is None else torch.full((1,), c["skip"], dtype=torch.int32, device=DEV)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=c["wd"], wd_mode=c["mode"],
              step=c["step"])
    d_t = None
    refused = False
    if seed % 4 == 3:                  # the grad scale and the step from device memory
        d_gs = torch.full((1,), c["gs"], dtype=torch.float32, device=DEV)
        table_len = [1, 7, 2500][seed // 4 % 3]      # shorter tables have no constants for t
        table = Z.adam_table(Z.adam_hparams(**hp), table_len, device=DEV)
        d_t = torch.full((1,), c["step"], dtype=torch.int64, device=DEV)
        d_status = torch.zeros(1, dtype=torch.int32, device=DEV)
        Z.zero_adam_shard_step_dev_t(d_reps, n, d_gs, table, d_t, d_status, d_p, d_m, d_v,
                                     wd_mode=c["mode"], out=d_out, skip=skip)
        refused = c["step"] > table_len and c["skip"] != 1
    elif seed % 2:                     # the grad scale read from device memory
        d_gs = torch.full((1,), c["gs"], dtype=torch.float32, device=DEV)
        Z.zero_adam_shard_step_dev_scale(d_reps, n, d_gs, d_p, d_m, d_v, Z.adam_hparams(**hp),
                                         out=d_out, skip=skip)
    else:
        Z.zero_adam_shard_step(d_reps, n, c["gs"], d_p, d_m, d_v, Z.adam_hparams(**hp), out=d_out,
                               skip=skip)
    torch.cuda.synchronize()
    if d_t is not None:
        assert int(d_t.item()) == c["step"] + (0 if c["skip"] == 1 or refused else 1)
        assert int(d_status.item()) == (Z.ZERO_DEV_T_OUT_OF_TABLE if refused else 0)
    skipped = c["skip"] == 1 or refused       # a refused update writes nothing, as a skipped one
    wp, wm, wv, wo = O.sharded_step(list(reps), c["rdt"], c["gs"], p, m, v, O.AdamHParams(**hp),
                                    c["odt"], skip=skipped)
    assert_bits_equal(bits32(d_p), f32_bits(wp), "master")
    assert_bits_equal(bits32(d_m), f32_bits(wm), "m")
    assert_bits_equal(bits32(d_v), f32_bits(wv), "v")
    if c["odt"]:
        got = bits16(full)
        fill = bits16(torch.full((1,), -2.0, dtype=_T16[c["odt"]], device=DEV))[0]
        assert (got[:o_out] == fill).all() and (got[o_out + n:] == fill).all(), "write outside the slot"
        if skipped:
            assert (got[o_out:o_out + n] == fill).all(), "skipped step wrote the slot"
        else:
            assert_bits_equal(got[o_out:o_out + n], wo, "out")


@pytest.mark.parametrize("seed", range(CASES // 2))
def test_random_reduce(seed):
    rng = np.random.default_rng(20_000 + seed)
    n = int(rng.choice([rng.integers(1, 600), rng.integers(600, 9000)]))
    R = int(rng.choice([1, 2, 5, 8, 16, 31, 64]))
    rdt = str(rng.choice(["f32", "f16", "bf16"]))
    off = int(rng.integers(0, 8)) if rng.random() < 0.5 else 0
    sq_scale = float(rng.choice([1.0, 2.0 ** -16, 0.37]))
    banner(f"random reduce seed={seed} n={n} R={R} {rdt} off={off}")
    reps = _draw_reps(rng, R, n, rdt)
    d_reps = [_placed(r, off, rdt) for r in reps]
    d_g = torch.empty(n, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    Z.zero_reduce_shard(d_reps, n, d_g, flag, parts, sq_scale)
    Z.zero_shard_sqnorm(None, n, sq_scale, parts, sq)
    torch.cuda.synchronize()
    acc = O.replica_sum(list(reps), rdt)
    assert_bits_equal(bits32(d_g), f32_bits(acc), "reduced gradient")
    assert int(flag.item()) == int(O.nonfinite_flag(acc))
    want = O.shard_sqnorm(acc, sq_scale)
    assert math.isclose(float(sq.item()), want, rel_tol=1e-10, abs_tol=0.0), (float(sq.item()), want)


@pytest.mark.parametrize("seed", range(CASES // 2))
def test_random_gather(seed):
    """ZeRO-3 gather: random shard counts and sizes, ranges, element sizes and source / output
    offsets; shards the range does not touch are passed as NULL."""
    rng = np.random.default_rng(30_000 + seed)
    nd = int(rng.choice([1, 2, 3, 8, 13, 64]))
    S = int(rng.choice([rng.integers(1, 50), rng.integers(50, 3000), rng.integers(3000, 70_000)]))
    eb = int(rng.choice([2, 4]))
    src_off, out_off = (int(x) if rng.random() < 0.5 else 0 for x in rng.integers(0, 8, 2))
    P = nd * S
    begin = int(rng.integers(0, P))
    count = int(rng.integers(0, P - begin + 1))
    banner(f"random gather seed={seed} nd={nd} S={S} eb={eb} [{begin}, {begin + count}) "
           f"offsets {src_off}/{out_off}")
    dt_np, dt_t = (np.int16, torch.int16) if eb == 2 else (np.int32, torch.int32)
    info = np.iinfo(dt_np)
    host = [rng.integers(info.min, info.max, S, endpoint=True).astype(dt_np) for _ in range(nd)]
    touched = set(range(begin // S, (begin + count - 1) // S + 1)) if count else set(range(nd))
    dev = [torch.from_numpy(np.concatenate([np.zeros(src_off, dt_np), h])).to(DEV)[src_off:]
           if r in touched else None for r, h in enumerate(host)]
    buf = torch.full((count + out_off + 3,), -5, dtype=dt_t, device=DEV)
    Z.zero_gather_params(dev, begin, count, buf[out_off:out_off + count])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:out_off] == -5).all() and (h[out_off + count:] == -5).all(), "write outside out"
    assert np.array_equal(h[out_off:out_off + count], O.gather_range(host, begin, count))
