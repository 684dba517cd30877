"""Even partition of the flattened model state over Nd data-parallel ranks.  TEST INFRASTRUCTURE.

What the pages fix: the model state (optimizer state in ZeRO-1, plus gradients in ZeRO-2, plus
parameters in ZeRO-3) is split evenly so that each rank holds 1/Nd of it and runs the optimizer on
its own subset only ([P1] "ZeRO 优化器的三个阶段深度对比", section 二; [P3] "ZeRO Optimization",
definition and core-operations lists; [P2] "ZeRO 优化器：把显存分着用", ZeRO Stage 1).

Readings where the pages are silent (padding, alignment, remainder placement, block layout):
  * contiguous blocks in rank order (rank r owns [r*S, (r+1)*S)), the chunking a reduce-scatter
    and an all-gather of a flat buffer use;
  * the shard size S is ceil(N/Nd) rounded up to a multiple of ``align_elems``; all padding sits
    at the tail of the flat space; padded length P = S*Nd;
  * N < Nd is allowed: the trailing ranks then own only padding (valid = 0);
  * sizes are unsigned 64-bit: a padded length of 2**64 or more is an overflow error.

Pinned by brute force in the CPU tests: ranks are disjoint, their union is [0, P), every shard has
the same size S, the valid parts tile [0, N) exactly, and pad < Nd*align_elems.
"""

from __future__ import annotations

from dataclasses import dataclass

U64_LIMIT = 1 << 64


@dataclass(frozen=True)
class Plan:
    n: int            # real parameter count N
    padded_n: int     # P = S * Nd
    shard_elems: int  # S, elements per rank, padding included
    pad: int          # P - N, all at the tail
    nd: int           # data-parallel degree
    align_elems: int  # S is a multiple of this


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def partition_plan(n: int, nd: int, align_elems: int = 1) -> Plan:
    """Shard size and padding for N flat elements over Nd ranks ([P1] section 二: 1/Nd per rank)."""
    if n < 0 or n >= U64_LIMIT:
        raise ValueError("n must be a non-negative 64-bit count")
    if nd < 1 or nd >= (1 << 32):
        raise ValueError("nd must be in [1, 2**32)")
    if align_elems < 1 or align_elems >= (1 << 32):
        raise ValueError("align_elems must be in [1, 2**32)")
    per_rank = _ceil_div(n, nd)                       # even split, remainder rounded up
    s = align_elems * _ceil_div(per_rank, align_elems)  # round the shard up to the alignment
    p = s * nd
    if p >= U64_LIMIT:
        raise OverflowError("padded length does not fit in 64 bits")
    return Plan(n=n, padded_n=p, shard_elems=s, pad=p - n, nd=nd, align_elems=align_elems)


def shard_range(plan: Plan, rank: int) -> tuple[int, int]:
    """(begin, valid) of rank ``rank``: it owns [begin, begin + S); the first ``valid`` are real."""
    if not 0 <= rank < plan.nd:
        raise ValueError("rank out of range")
    begin = rank * plan.shard_elems
    valid = min(plan.shard_elems, max(0, plan.n - begin))
    return begin, valid
