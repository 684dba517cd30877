"""ZeRO-3 parameter gather for one layer.  TEST INFRASTRUCTURE.

[P1] "ZeRO 优化器的三个阶段深度对比", section 三, [P2] "ZeRO 优化器：把显存分着用", ZeRO Stage 3, and
[P3] "ZeRO Optimization", core-operations list: with parameters sharded, each layer's full
parameters are rebuilt from every rank's shard (an all-gather) right before the layer runs, and the
parts other ranks own are released after use. With the even contiguous partition, rank r holds flat
elements [r*S, (r+1)*S), so the gathered flat space is the rank shards laid end to end, and a
layer's parameters are the slice of it that the layer occupies.

The definition is written out here: concatenate the shards in rank order, take the slice.
Pinned in the CPU tests by a per-element brute force (flat index j lives in shard j // S at
offset j % S) and by the partition's union property.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def gather_range(shards: Sequence[np.ndarray], begin: int, count: int) -> np.ndarray:
    """flat[begin : begin + count] of the rank shards laid end to end (all the same length S)."""
    if len(shards) == 0:
        raise ValueError("at least one shard")
    S = len(shards[0])
    if any(len(s) != S for s in shards):
        raise ValueError("shards must have equal length")
    if begin < 0 or count < 0 or begin + count > S * len(shards):
        raise ValueError("range outside the gathered space")
    flat = np.concatenate([np.asarray(s) for s in shards])
    return flat[begin:begin + count].copy()
