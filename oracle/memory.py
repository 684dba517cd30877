"""Per-rank model-state memory for data parallelism and ZeRO stages 1-3.  TEST INFRASTRUCTURE.

[P1] "ZeRO 优化器的三个阶段深度对比", section 二, gives an estimator: per parameter, 2 bytes of
16-bit parameters, 2 bytes of 16-bit gradients and 12 bytes of Adam state (fp32 copy, m, v); plain
data parallelism keeps all three whole on every rank, ZeRO-1 divides the optimizer state by Nd,
ZeRO-2 also the gradients, ZeRO-3 also the parameters; results in units of 1024**3 bytes. The same
split is stated in section 一 and in [P3] "ZeRO Optimization", stages list. This module restates
that rule in its own form: a table of which component each stage shards.

``stage_bytes_exact`` is the integer variant for a concrete plan: a sharded component costs
S (the padded shard size) elements per rank instead of N/Nd.

``stage_comm_bytes`` is the other side of that trade: the bytes one rank sends per step under
each stage, for ring collectives over the same plan.

``choose_stage`` is the stage-choice rule of [P1] section 四 (a decision tree: a card that can hold
the whole model takes ZeRO-1; one that cannot, but can hold parameters and gradients, takes ZeRO-2;
one that cannot even hold the parameters needs ZeRO-3, with optimizer-state offload advised). The
page does not say against which budget "hold" is judged; the reading here is: the smallest stage of
1..3 whose exact per-rank model-state bytes fit in the caller's usable byte budget (card capacity
less what the caller reserves for activations and buffers), and ZeRO-3 plus the offload advice when
none fits. Pinned to the page's three examples (7B, 13B, 70B on an 80 GB card) under a stated
reading of their unstated data-parallel degree and reserve.
"""

from __future__ import annotations

from dataclasses import dataclass

from .partition import Plan

GIB = 1024 ** 3

# stage -> which of (optimizer state, gradients, parameters) is divided over the Nd ranks
STAGES = {
    "DP": (False, False, False),
    "ZeRO-1": (True, False, False),
    "ZeRO-2": (True, True, False),
    "ZeRO-3": (True, True, True),
}


@dataclass(frozen=True)
class MemoryEstimation:
    optimizer_states: float  # GiB per rank
    gradients: float
    parameters: float
    total: float


def estimate_memory_per_gpu(num_params: float, dp_degree: int, bytes_per_param: int = 2,
                            bytes_per_opt_state: int = 12) -> dict[str, MemoryEstimation]:
    """Per-rank GiB of each model-state component for every stage (gradients use the 16-bit size)."""
    per_param = (bytes_per_opt_state, bytes_per_param, bytes_per_param)  # opt, grad, param
    out = {}
    for stage, sharded in STAGES.items():
        comp = [num_params * b / (dp_degree if s else 1) for b, s in zip(per_param, sharded)]
        out[stage] = MemoryEstimation(comp[0] / GIB, comp[1] / GIB, comp[2] / GIB, sum(comp) / GIB)
    return out


def stage_bytes_exact(plan: Plan, stage: int, param_b: int = 2, grad_b: int = 2,
                      opt_b: int = 12) -> tuple[int, int, int, int]:
    """(optimizer, gradient, parameter, total) bytes on one rank, integers; stage 0 = DP, 1..3."""
    names = ("DP", "ZeRO-1", "ZeRO-2", "ZeRO-3")
    if not 0 <= stage <= 3:
        raise ValueError("stage must be 0..3")
    sharded = STAGES[names[stage]]
    comp = [b * (plan.shard_elems if s else plan.n)
            for b, s in zip((opt_b, grad_b, param_b), sharded)]
    total = sum(comp)
    if total >= 1 << 64:
        raise OverflowError("byte count does not fit in 64 bits")
    return comp[0], comp[1], comp[2], total


def stage_comm_bytes(plan: Plan, stage: int, param_b: int = 2,
                     grad_b: int = 2) -> tuple[int, int, int]:
    """(gradient, parameter, total) bytes one rank sends per training step; stage 0 = DP, 1..3.

    [P1] section 一 and [P3] stages list: ZeRO-1 and ZeRO-2 move as much as plain data parallelism,
    ZeRO-3 about 1.5 times as much; [P1] section 二 puts the volume of each of the first two at
    about 2N, and section 三 traces ZeRO-3's extra to all-gathering every layer's parameters.
    Reading: collectives run as rings over the plan's padded buffer of Nd*S elements, so one
    reduce-scatter or one all-gather sends (Nd-1)*S elements per rank, and an all-reduce is one of
    each. Plain DP all-reduces the gradients; ZeRO-1/2 reduce-scatter the gradients and all-gather
    the updated parameters; ZeRO-3 all-gathers the parameters twice (forward and backward) and
    reduce-scatters the gradients ([P1] section 三 says all-gather for the gradients in the
    backward; the reading follows its section 二 and [P3], which say reduce-scatter).
    """
    if not 0 <= stage <= 3:
        raise ValueError("stage must be 0..3")
    one = (plan.nd - 1) * plan.shard_elems            # elements one rank sends in one ring pass
    grad_passes, param_passes = ((2, 0), (1, 1), (1, 1), (1, 2))[stage]
    g, w = grad_passes * one * grad_b, param_passes * one * param_b
    if g + w >= 1 << 64:
        raise OverflowError("byte count does not fit in 64 bits")
    return g, w, g + w


def choose_stage(plan: Plan, usable_bytes: int, param_b: int = 2, grad_b: int = 2,
                 opt_b: int = 12) -> tuple[int, bool, tuple[int, int, int, int]]:
    """(stage 1..3, offload advised, that stage's per-rank bytes) for a budget of usable bytes."""
    if usable_bytes < 0:
        raise ValueError("usable_bytes must be >= 0")
    for stage in (1, 2, 3):
        b = stage_bytes_exact(plan, stage, param_b, grad_b, opt_b)
        if b[3] <= usable_bytes:
            return stage, False, b
    return 3, True, stage_bytes_exact(plan, 3, param_b, grad_b, opt_b)
