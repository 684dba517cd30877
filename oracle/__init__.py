"""CPU oracle for one data-parallel rank's sharded ZeRO optimizer step.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import or call anything in this package. The product path
(the HIP library and its Python binding) never imports it and shares no code with it.

It is plain and slow on purpose: numpy only, whole arrays, one ufunc per arithmetic operation,
so every fp32 operation is rounded once (IEEE round-to-nearest-even) in the order written, and
scalars are formed in Python floats (fp64) and rounded once to fp32.

Sources (cited by title and section; the pages were read as data, nothing is quoted):
  [P1] "ZeRO 优化器的三个阶段深度对比：显存节省与通信开销的量化分析" (wmrh.cn/news/520095),
       sections 一 .. 五, with a Python memory estimator in section 二.
  [P2] "ZeRO 优化器：把显存“分”着用" (5688vip.com), sections "ZeRO Stage 1" .. "ZeRO-Offload".
  [P3] "ZeRO Optimization（零冗余优化）" glossary (ai-master.cc): definition, core operations,
       stages, comparisons, limitations.
  The pages give no update equations, no loss scaling, clipping or overflow handling; where this
  oracle fills such a gap it says which reading it takes.

Modules:
  partition  even contiguous split of the flat padded parameter space          [P1 二; P3 stages]
  adam       replica sum, non-finite flag, squared norm, clip coefficient,
             Adam/AdamW update and the full per-rank step                          [P1 二; P2 Stage 1/2]
  cast       fp32 -> bf16 / fp16 round-to-nearest-even (bit patterns as uint16)  [P1 一; P3 comparisons]
  gather     ZeRO-3 gather of one layer's parameters from the rank shards         [P1 三; P3 core operations]
  memory     per-stage model-state bytes per rank (DP, ZeRO-1/2/3), the bytes a
             rank sends per step under each stage, and the stage-choice rule  [P1 一/二/三/四; P3 stages]

Parity status of each function is stated in its docstring. The clip coefficient has no page; its
reading is pinned against torch.nn.utils.clip_grad_norm_, a library implementation of the rule.
"""

from .partition import Plan, partition_plan, shard_range
from .cast import cast_bf16_rne, cast_fp16_rne, widen_bf16, widen_fp16
from .adam import (
    AdamHParams,
    AdamScalars,
    adam_scalars,
    adam_update,
    replica_sum,
    nonfinite_flag,
    shard_sqnorm,
    clip_coefficient,
    sharded_step,
    unsharded_step,
)
from .gather import gather_range
from .memory import (MemoryEstimation, estimate_memory_per_gpu, stage_bytes_exact, stage_comm_bytes, STAGES,
                     choose_stage)

__all__ = [
    "Plan", "partition_plan", "shard_range",
    "cast_bf16_rne", "cast_fp16_rne", "widen_bf16", "widen_fp16",
    "AdamHParams", "AdamScalars", "adam_scalars", "adam_update", "replica_sum",
    "nonfinite_flag", "shard_sqnorm", "clip_coefficient", "sharded_step", "unsharded_step",
    "gather_range",
    "MemoryEstimation", "estimate_memory_per_gpu", "stage_bytes_exact", "stage_comm_bytes", "STAGES",
    "choose_stage",
]
