"""One rank's sharded optimizer step, written out plainly.  TEST INFRASTRUCTURE.

The step the pages describe for ZeRO-1/2 ([P1] "ZeRO 优化器的三个阶段深度对比", section 二;
[P2] "ZeRO 优化器：把显存分着用", ZeRO Stage 1 and Stage 2; [P3] "ZeRO Optimization", core
operations): gradients are summed over the data-parallel replicas and only the rank's part is kept
(the reduce half of a reduce-scatter); the rank runs Adam on its own parameter subset with its own
optimizer state (fp32 parameter copy, first moment m, second moment v: 12 bytes per parameter);
the updated parameters are then gathered to every rank in 16-bit form.

Readings (the pages name Adam and its state but print no equations, and say nothing of loss
scaling, overflow or clipping):
  * replica sum: a sum, not a mean, in ascending replica order with an fp32 accumulator, each
    replica widened exactly to fp32 first. A mean is the same sum with grad_scale = 1/Nd.
  * Adam: Kingma and Ba with bias correction, t counted from 1, eps added after the
    bias-corrected square root; AdamW decay is decoupled and applied to p before the Adam step;
    L2 mode adds wd*p to the gradient instead. The fp32 operation order is fixed (see
    ``adam_update``) so that another implementation can reproduce it bit for bit.
  * overflow: the whole step is skipped when any summed gradient element is not finite.
  * squared norm: sum over the shard of (acc_i * sq_scale)^2 with fp64 terms, padding included.
  * clip coefficient: min(1, max_norm / (sqrt(total_sq) + 1e-6)) in fp64. No page defines it; the
    reading is the usual global-norm rule, pinned against torch.nn.utils.clip_grad_norm_ (which
    forms its own norm and coefficient) in the tests.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Sequence

import numpy as np

from .cast import cast_bf16_rne, cast_fp16_rne, widen_bf16, widen_fp16

F32 = np.float32


@dataclass(frozen=True)
class AdamHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    wd_mode: str = "adamw"   # "adamw" (decoupled) or "l2" (added to the gradient)
    step: int = 1            # t >= 1, this step included


@dataclass(frozen=True)
class AdamScalars:
    b1: np.float32
    b2: np.float32
    c1: np.float32    # 1 - beta1
    c2: np.float32    # 1 - beta2
    ss: np.float32    # lr / (1 - beta1^t)
    bc: np.float32    # sqrt(1 - beta2^t)
    e: np.float32     # eps
    dec: np.float32   # 1 - lr * wd   (AdamW)
    w: np.float32     # wd            (L2)


def adam_scalars(hp: AdamHParams) -> AdamScalars:
    """fp32 step constants: each is formed in fp64 and rounded to fp32 once."""
    if hp.step < 1:
        raise ValueError("step counts from 1")
    t = float(hp.step)
    return AdamScalars(
        b1=F32(hp.beta1),
        b2=F32(hp.beta2),
        c1=F32(1.0 - hp.beta1),
        c2=F32(1.0 - hp.beta2),
        ss=F32(hp.lr / (1.0 - math.pow(hp.beta1, t))),
        bc=F32(math.sqrt(1.0 - math.pow(hp.beta2, t))),
        e=F32(hp.eps),
        dec=F32(1.0 - hp.lr * hp.weight_decay),
        w=F32(hp.weight_decay),
    )


def _widen(rep: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return widen_bf16(rep)
    if dtype == "f16":
        return widen_fp16(rep)
    if dtype == "f32":
        return np.ascontiguousarray(rep, dtype=np.float32)
    raise ValueError(f"unknown replica dtype {dtype!r}")


def replica_sum(reps: Sequence[np.ndarray], dtype: str) -> np.ndarray:
    """acc = rep_0 + rep_1 + ... + rep_{R-1}, left to right, fp32, each add rounded.

    Replicas are uint16 bit patterns for "bf16"/"f16" and float32 for "f32". This is the
    reduction half of the gradient reduce-scatter, done over local copies ([P1] section 二).
    """
    if len(reps) == 0:
        raise ValueError("at least one replica")
    acc = _widen(reps[0], dtype).copy()
    with np.errstate(over="ignore", invalid="ignore"):   # inf and NaN are defined results here
        for k in range(1, len(reps)):
            acc = acc + _widen(reps[k], dtype)
    return acc


def nonfinite_flag(acc: np.ndarray) -> bool:
    """True when any summed gradient element is +-inf or NaN (overflow-skip reading)."""
    return not bool(np.isfinite(acc).all())


def shard_sqnorm(acc: np.ndarray, sq_scale: float = 1.0, chunk: int = 1 << 20) -> float:
    """sum_i (fp64(acc_i) * sq_scale)^2 over the shard.

    Terms are formed in fp64 (exact when sq_scale is a power of two: a 24-bit significand squared
    fits in 53 bits). Chunks of 2**20 terms are summed pairwise by numpy and the chunk sums are
    added with math.fsum, so the result is within a few fp64 ulps of the exact sum of the terms.
    """
    a = np.ascontiguousarray(acc, dtype=np.float32).reshape(-1)
    s = np.float64(sq_scale)
    parts = []
    for i in range(0, a.size, chunk):
        t = a[i:i + chunk].astype(np.float64) * s
        parts.append(float(np.sum(t * t)))
    return math.fsum(parts)


def clip_coefficient(total_sq: float, max_norm: float = 1.0, eps: float = 1e-6) -> float:
    """min(1, max_norm / (||g|| + eps)) in IEEE fp64: a zero norm with eps = 0 divides to +inf
    (coefficient 1), an infinite norm gives 0, and a NaN quotient gives 1. No page defines
    clipping; this is the global-norm rule read for the clipped step, pinned against
    torch.nn.utils.clip_grad_norm_ on fp64 gradients (exact norms below, at and above max_norm,
    tiny and huge norms, random gradients) and by planted mistakes that those pins catch."""
    with np.errstate(divide="ignore", invalid="ignore"):
        q = float(np.float64(max_norm) / (np.sqrt(np.float64(total_sq)) + np.float64(eps)))
    return min(1.0, q)


def adam_update(p: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray,
                sc: AdamScalars, wd_mode: str = "adamw"):
    """One Adam/AdamW update in fp32; every line is one rounded operation per element.

    Returns new (p, m, v); the inputs are not modified.
    """
    if wd_mode == "l2":
        g = g + sc.w * p                      # L2: decay folded into the gradient
    elif wd_mode != "adamw":
        raise ValueError(f"unknown wd_mode {wd_mode!r}")
    m = sc.b1 * m + sc.c1 * g                 # first moment
    v = sc.b2 * v + sc.c2 * (g * g)           # second moment
    den = np.sqrt(v) / sc.bc + sc.e           # bias-corrected sqrt(v_hat) + eps
    if wd_mode == "adamw":
        p = p * sc.dec                        # decoupled decay (dec = 1 when wd = 0)
    p = p - sc.ss * (m / den)                 # ss carries the 1/(1 - beta1^t) correction
    return p, m, v


def _cast(p: np.ndarray, out_dtype: str | None):
    if out_dtype is None:
        return None
    if out_dtype == "bf16":
        return cast_bf16_rne(p)
    if out_dtype == "f16":
        return cast_fp16_rne(p)
    raise ValueError(f"unknown out dtype {out_dtype!r}")


def sharded_step(reps: Sequence[np.ndarray], rep_dtype: str, grad_scale: float,
                 master: np.ndarray, m: np.ndarray, v: np.ndarray, hp: AdamHParams,
                 out_dtype: str | None = "bf16", skip: bool = False):
    """The rank's whole step on its shard: sum replicas, scale, Adam, cast for the slot.

    Returns (master', m', v', out16 or None). With ``skip`` the state comes back unchanged and
    no 16-bit output is produced (the caller's slot keeps its old contents).
    """
    if skip:
        return master.copy(), m.copy(), v.copy(), None
    acc = replica_sum(reps, rep_dtype)
    g = acc * F32(grad_scale)
    p2, m2, v2 = adam_update(np.asarray(master, np.float32), np.asarray(m, np.float32),
                             np.asarray(v, np.float32), g, adam_scalars(hp), hp.wd_mode)
    return p2, m2, v2, _cast(p2, out_dtype)


def unsharded_step(grad_full: np.ndarray, master_full: np.ndarray, m_full: np.ndarray,
                   v_full: np.ndarray, hp: AdamHParams, grad_scale: float = 1.0,
                   out_dtype: str | None = "bf16"):
    """Plain data-parallel Adam over the whole flat buffer (one fp32 gradient, no sharding).

    The pages say ZeRO changes only where the state is stored, not the computation ([P3] "ZeRO
    Optimization", comparisons and limitations), so the union of the rank shards' results must
    equal this, element for element.
    """
    g = np.asarray(grad_full, np.float32) * F32(grad_scale)
    p2, m2, v2 = adam_update(np.asarray(master_full, np.float32), np.asarray(m_full, np.float32),
                             np.asarray(v_full, np.float32), g, adam_scalars(hp), hp.wd_mode)
    return p2, m2, v2, _cast(p2, out_dtype)
