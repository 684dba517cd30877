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
