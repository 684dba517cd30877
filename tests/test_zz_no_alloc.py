"""The entry point that allocates nothing (zero_reduce_shard_static) against the calls it stands
for (zero_reduce_shard with a caller's partials buffer, then zero_shard_sqnorm): gradient, flag and
squared norm bit for bit, on two calls in a row with the second smaller, so the scratch the
library keeps between calls cannot leak into the second result."""

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, assert_bits_equal, banner, bits32, dev_rep, f32_bits

pytestmark = pytest.mark.gpu


def _reps(rng, R, n, dtype, scale):
    x = (rng.standard_normal((R, n)) * 1e-3).astype(np.float32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return (x * np.float32(scale)).astype(np.float16).view(np.uint16)


def _both(d_reps, n, sq_scale):
    """(gradient, flag, norm) of the static entry point and of the workspace pair, each fresh."""
    out = []
    for static in (True, False):
        g = torch.full((n,), float("nan"), device=DEV)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        sq = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        if static:
            Z.zero_reduce_shard_static(d_reps, n, g, flag, sq, sq_scale)
        else:
            parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
            Z.zero_reduce_shard(d_reps, n, g, flag, parts, sq_scale)
            Z.zero_shard_sqnorm(None, n, sq_scale, parts, sq)
        torch.cuda.synchronize()
        out.append((bits32(g), int(flag.item()), float(sq.item())))
    return out


@pytest.mark.parametrize("dtype,R", [("f16", 16), ("bf16", 8), ("bf16", 3)])
def test_static_scratch_equals_workspace_calls(dtype, R):
    rng = np.random.default_rng(R)
    scale = 2.0 ** 8 if dtype == "f16" else 1.0
    for n in (300_000 + 77, 9_001):                 # the second call is smaller
        banner(f"no-alloc reduce {dtype} R={R} n={n}")
        reps = _reps(rng, R, n, dtype, scale)
        d_reps = [dev_rep(r, dtype) for r in reps]
        (g_s, f_s, sq_s), (g_w, f_w, sq_w) = _both(d_reps, n, 1.0 / scale)
        assert_bits_equal(g_s, g_w, "gradient")
        assert f_s == f_w == 0
        assert sq_s == sq_w                          # the same partials, the same fixed order
        acc = O.replica_sum(list(reps), dtype)
        assert_bits_equal(g_s, f32_bits(acc), "gradient vs oracle")
        want = O.shard_sqnorm(acc, 1.0 / scale)
        assert abs(sq_s - want) <= 1e-10 * want


def test_static_scratch_flag_and_norm_only():
    """Only the flag and the norm requested (no gradient written), with an infinity injected in
    the first call and a clean, smaller second call."""
    rng = np.random.default_rng(5)
    for n, bad in ((70_000, True), (1_000, False)):
        reps = _reps(rng, 4, n, "f16", 1.0)
        if bad:
            reps[2][n // 3] = 0x7C00                  # +inf in binary16
        d_reps = [dev_rep(r, "f16") for r in reps]
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        sq = torch.empty(1, dtype=torch.float64, device=DEV)
        Z.zero_reduce_shard_static(d_reps, n, None, flag, sq, 1.0)
        parts = torch.empty(Z.zero_sq_partials_len(n), dtype=torch.float64, device=DEV)
        sq_w = torch.empty(1, dtype=torch.float64, device=DEV)
        Z.zero_reduce_shard(d_reps, n, None, None, parts, 1.0)
        Z.zero_shard_sqnorm(None, n, 1.0, parts, sq_w)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(bad)
        a, b = float(sq.item()), float(sq_w.item())
        assert (a == b) or (np.isnan(a) and np.isnan(b)) or (np.isinf(a) and a == b)


def test_static_scratch_edges():
    """An empty shard writes a zero norm; a call that asks for no norm uses no scratch and still
    gives the gradient; a ragged size shorter than one tile; each checked against the workspace
    pair."""
    rng = np.random.default_rng(9)
    reps = _reps(rng, 5, 77, "bf16", 1.0)
    d_reps = [dev_rep(r, "bf16") for r in reps]
    sq = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    Z.zero_reduce_shard_static(d_reps, 0, None, None, sq, 1.0)
    torch.cuda.synchronize()
    assert float(sq.item()) == 0.0
    g = torch.full((77,), float("nan"), device=DEV)
    Z.zero_reduce_shard_static(d_reps, 77, g, None, None, 1.0)
    torch.cuda.synchronize()
    assert_bits_equal(bits32(g), f32_bits(O.replica_sum(list(reps), "bf16")), "gradient without a norm")
    (g_s, f_s, sq_s), (g_w, f_w, sq_w) = _both(d_reps, 77, 1.0)
    assert_bits_equal(g_s, g_w, "ragged gradient")
    assert sq_s == sq_w and f_s == f_w == 0
