"""Device memory for an arena: zero_arena_alloc / zero_arena_free through the binding's arena(),
which hands the allocation to torch. Views land at the offsets zero_arena_layout gives, hold what
is written to them, and the memory is released when the last tensor on it dies."""

import gc

import pytest
import torch

import zero_partition_plan_amd as Z
from gpu_util import DEV, banner

pytestmark = pytest.mark.gpu


def _specs(n):
    return [("rep0", n, torch.bfloat16, 0, 0), ("rep1", n, torch.bfloat16, 0, 0),
            ("master", n, torch.float32, 1, 0), ("m", n, torch.float32, 1, 0),
            ("slot", n + 7, torch.bfloat16, 0, 5)]


def test_arena_views_and_offsets():
    n = 1 << 20
    banner("arena views")
    storage, views = Z.arena(_specs(n), device=DEV)
    assert storage.is_cuda and storage.dtype == torch.uint8
    assert isinstance(storage.zero_arena_contiguous, bool)
    offs, total = Z.zero_arena_layout([(c * torch.empty(0, dtype=t).element_size(),
                                        h * torch.empty(0, dtype=t).element_size(), g,
                                        torch.empty(0, dtype=t).element_size())
                                       for _, c, t, g, h in _specs(n)])
    assert storage.numel() == total
    for (name, c, t, _, _), o in zip(_specs(n), offs):
        v = views[name]
        assert v.dtype == t and v.numel() == c and v.data_ptr() - storage.data_ptr() == o, name
    for i, name in enumerate(views):
        views[name].fill_(float(i + 1))
    torch.cuda.synchronize()
    for i, name in enumerate(views):
        assert bool((views[name] == float(i + 1)).all()), name
    del storage, views
    gc.collect()


def test_arena_memory_is_released():
    nbytes = 6 << 30
    banner("arena release")
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    storage, views = Z.arena([("a", nbytes // 4, torch.float32, 0, 0)], device=DEV)
    views["a"][:1024].fill_(3.0)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 >= nbytes - (64 << 20)
    del storage, views
    gc.collect()
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert free2 >= free0 - (256 << 20), (free0, free2)


def test_arena_alloc_edges():
    assert Z.zero_arena_alloc(0) == (None, False)
    Z.zero_arena_free(None)
    p, contiguous = Z.zero_arena_alloc(1 << 20)
    assert p and isinstance(contiguous, bool)
    torch.cuda.synchronize()
    Z.zero_arena_free(p)
    with pytest.raises(Z.ZeroError):
        Z.zero_arena_alloc(1 << 62)                    # more than any device holds


@pytest.mark.parametrize("nd", [3, 8])
def test_step_on_arena_views_with_slot_offsets(nd):
    """Every rank of a ragged plan steps on arena views, its slot found inside the gathered buffer
    at r*S (the layout's hot offset): the slot equals the oracle's cast, bit for bit, and the rest
    of the buffer is untouched."""
    import numpy as np

    import oracle as O
    from gpu_util import assert_bits_equal, bits16, bits32, f32_bits

    n = 1_234_567
    plan = Z.zero_partition_plan(n, nd)
    S = plan.shard_elems
    rng = np.random.default_rng(nd)
    for r in range(nd):
        begin, valid = Z.zero_shard_range(plan, r)
        specs = [(f"rep{k}", S, torch.bfloat16, 0, 0) for k in range(2)]
        specs += [("full", plan.padded_n, torch.bfloat16, 0, begin), ("master", S, torch.float32, 1, 0),
                  ("m", S, torch.float32, 1, 0), ("v", S, torch.float32, 1, 0)]
        storage, a = Z.arena(specs, device=DEV)
        reps = (rng.standard_normal((2, S)).astype(np.float32) * np.float32(1e-3)).view(np.uint32) >> 16
        reps = reps.astype(np.uint16)
        reps[:, valid:] = 0
        master = (rng.standard_normal(S) * 0.02).astype(np.float32)
        master[valid:] = 0
        for k in range(2):
            a[f"rep{k}"].copy_(torch.from_numpy(reps[k].view(np.int16)).view(torch.bfloat16))
        a["master"].copy_(torch.from_numpy(master))
        a["m"].zero_()
        a["v"].zero_()
        a["full"].fill_(-9.0)
        hp = dict(lr=1e-3, weight_decay=0.01, step=1)
        Z.zero_adam_shard_step([a["rep0"], a["rep1"]], S, 1.0, a["master"], a["m"], a["v"],
                               Z.adam_hparams(**hp), out=a["full"][begin:begin + S])
        torch.cuda.synchronize()
        z = np.zeros(S, np.float32)
        wp, _, _, wo = O.sharded_step(list(reps), "bf16", 1.0, master, z, z, O.AdamHParams(**hp), "bf16")
        assert_bits_equal(bits32(a["master"]), f32_bits(wp), f"master r={r}")
        full = bits16(a["full"])
        assert_bits_equal(full[begin:begin + S], wo, f"slot r={r}")
        fill = O.cast_bf16_rne(np.float32([-9.0]))[0]
        assert (full[:begin] == fill).all() and (full[begin + S:] == fill).all(), f"outside r={r}"
        del storage, a
