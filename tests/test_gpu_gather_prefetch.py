"""ZeRO-3's prefetch pipeline on two streams, checked for races: layer i+1 is gathered on a second
stream while layer i is read on the current one, two layer buffers alternate, events order each
read after its gather and each gather after the previous read of its buffer. Every layer's read
(a copy taken after a deliberately slow matmul, so a gather that ran ahead would be caught) must
equal the oracle's gather of that range."""

import numpy as np
import pytest
import torch

import oracle as O
import zero_partition_plan_amd as Z
from gpu_util import DEV, banner

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nd,seed", [(8, 0), (3, 1), (64, 2)])
def test_prefetch_pipeline_reads_each_layer_whole(nd, seed):
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(1, 3_000_000, 12)] + [4096 * 700, 5]
    P = sum(sizes)
    S = -(-P // nd)
    banner(f"prefetch pipeline nd={nd} layers={len(sizes)} P={P}")
    flat = rng.integers(-(1 << 15), 1 << 15, S * nd).astype(np.int16)
    host = [flat[r * S:(r + 1) * S] for r in range(nd)]
    shards = [torch.from_numpy(h.copy()).to(DEV) for h in host]
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    bufs = [torch.empty(max(sizes), dtype=torch.int16, device=DEV) for _ in range(2)]
    seen = [None] * len(sizes)
    x = torch.randn(512, 2048, device=DEV)
    w = torch.randn(2048, 2048, device=DEV)
    comp, gat = torch.cuda.current_stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event(), torch.cuda.Event()]
    free = [torch.cuda.Event(), torch.cuda.Event()]

    gat.wait_stream(comp)
    Z.zero_gather_params(shards, starts[0], sizes[0], bufs[0], stream=gat)
    ready[0].record(gat)
    for i in range(len(sizes)):
        if i + 1 < len(sizes):
            if i >= 1:
                gat.wait_event(free[(i + 1) % 2])
            Z.zero_gather_params(shards, starts[i + 1], sizes[i + 1], bufs[(i + 1) % 2], stream=gat)
            ready[(i + 1) % 2].record(gat)
        comp.wait_event(ready[i % 2])
        for _ in range(4):                      # slow the reader down
            x = torch.tanh(x @ w) * 0.5
        seen[i] = bufs[i % 2][:sizes[i]].clone()
        free[i % 2].record(comp)
    comp.wait_stream(gat)
    torch.cuda.synchronize()
    for i, (a, n) in enumerate(zip(starts, sizes)):
        assert np.array_equal(seen[i].cpu().numpy(), O.gather_range(host, a, n)), f"layer {i}"
