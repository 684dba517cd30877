"""Which arrays one rank's step touches, and which of them a kernel walks together, for placing
them in one arena (``zero_partition_plan_amd.arena``).

Each entry is (name, numel, dtype, group, hot_elem). Arrays in one group are read or written at the
same element index by one kernel: the replica rows and the 16-bit output of the fused pass; the
fp32 state (and the two-pass gradient) of the update. hot_elem is where that walk starts inside the
array: rank r's slot inside a gathered buffer starts at r*S. Names and sizes only; nothing here
computes any part of the step.
"""

from __future__ import annotations

import torch

from .shapes import Workload

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
REPLICAS, STATE, SLOT = 0, 1, 2


def step_arrays(w: Workload, S: int, begin: int, padded_n: int, two_pass: bool = False):
    """The arrays of one rank's step on workload ``w`` (shard of S elements starting at ``begin``).

    Fused single pass: replica rows and the gathered 16-bit buffer (walked from the rank's slot)
    form one group, master/m/v another. Two-pass: replica rows; master/m/v and the fp32 gradient;
    the slot alone. With a replica window, rows hold the window and the slot is its own array.
    """
    rows = S if w.window is None else w.window
    out_dt = _DT[w.out_dtypes[0]]
    arr = [(f"rep{k}", rows, _DT[w.rep_dtype], REPLICAS, 0) for k in range(w.reps)]
    fused_full = not two_pass and w.window is None
    if fused_full:
        arr.append(("full", padded_n, out_dt, REPLICAS, begin))
    arr += [("master", S, torch.float32, STATE, 0), ("m", S, torch.float32, STATE, 0),
            ("v", S, torch.float32, STATE, 0)]
    if two_pass:
        arr.append(("g", S, torch.float32, STATE, 0))
    if not fused_full:
        arr.append(("slot", S, out_dt, SLOT, 0))
    return arr
