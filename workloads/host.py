"""numpy generators for the workloads small enough to draw on the CPU.

Draw order per rank is fixed (master, then replicas 0..R-1, then the injected-inf mask, then warm
m and v), all from ``numpy.random.default_rng(seed)`` (PCG64). Padding positions (flat index >= N)
hold 0 in the master copy and in every replica, as a padded flat gradient buffer would.

16-bit replicas are returned as uint16 bit patterns: bf16 by truncating an fp32 draw to its top
16 bits, fp16 by numpy's float16 conversion of (draw * loss_scale). These are input recipes, not the
step's casts.
"""

from __future__ import annotations

import math

import numpy as np

from .shapes import Workload, init_ranges


def master_shard(w: Workload, begin: int, size: int, rng: np.random.Generator) -> np.ndarray:
    """fp32 master copy for flat range [begin, begin + size)."""
    x = rng.standard_normal(size, dtype=np.float32) * np.float32(w.master_std)
    if w.model is not None:
        end = begin + size
        for s, e, kind in init_ranges(w.model):
            lo, hi = max(s, begin), min(e, end)
            if lo < hi:
                x[lo - begin:hi - begin] = 1.0 if kind == "one" else 0.0
    if begin + size > w.n:
        x[max(0, w.n - begin):] = 0.0
    return x


def _to_rep_dtype(x: np.ndarray, w: Workload) -> np.ndarray:
    if w.rep_dtype == "f32":
        return x
    if w.rep_dtype == "bf16":
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if w.rep_dtype == "f16":
        return (x * np.float32(w.loss_scale)).astype(np.float16).view(np.uint16)
    raise ValueError(w.rep_dtype)


def replicas(w: Workload, size: int, valid: int, rng: np.random.Generator,
             reps: int | None = None) -> np.ndarray:
    """[R, size] replica slices; elements at index >= valid (padding) are 0."""
    r = w.reps if reps is None else reps
    out = []
    for _ in range(r):
        x = rng.standard_normal(size, dtype=np.float32) * np.float32(w.rep_std)
        x[valid:] = 0.0
        out.append(_to_rep_dtype(x, w))
    arr = np.stack(out)
    if w.inf_rate > 0.0:
        mask = rng.random(arr.shape) < w.inf_rate
        mask[:, valid:] = False
        inf_bits = {"f32": None, "bf16": 0x7F80, "f16": 0x7C00}[w.rep_dtype]
        if inf_bits is None:
            arr[mask] = np.inf
        else:
            arr[mask] = inf_bits
    return arr


def warm_state(w: Workload, size: int, valid: int, rng: np.random.Generator):
    """m, v drawn at the scale they would have after ``w.warm_steps`` steps (zeros if none).

    With iid N(0, sg) gradients, an EMA with factor b after k steps from 0 has standard deviation
    sg*(1-b)*sqrt((1-b^(2k))/(1-b^2)); v is drawn as (1-b2^k)*sg^2*U(0.5, 1.5). sg is the std of the
    summed gradient (rep_std * sqrt(R)).
    """
    m = np.zeros(size, np.float32)
    v = np.zeros(size, np.float32)
    k = w.warm_steps
    if k > 0:
        sg = w.rep_std * math.sqrt(w.reps)
        sm = sg * (1 - w.beta1) * math.sqrt((1 - w.beta1 ** (2 * k)) / (1 - w.beta1 ** 2))
        m[:] = rng.standard_normal(size, dtype=np.float32) * np.float32(sm)
        v[:] = (rng.random(size, dtype=np.float32) + np.float32(0.5)) * np.float32((1 - w.beta2 ** k) * sg * sg)
        m[valid:] = 0.0
        v[valid:] = 0.0
    return m, v


def rank_inputs(w: Workload, begin: int, size: int, valid: int, seed_offset: int = 0):
    """All inputs of one rank's step: dict(master, m, v, reps)."""
    rng = np.random.default_rng(w.seed + seed_offset)
    master = master_shard(w, begin, size, rng)
    reps = replicas(w, size, valid, rng)
    m, v = warm_state(w, size, valid, rng)
    return {"master": master, "m": m, "v": v, "reps": reps}


def flat_inputs(w: Workload, padded_n: int):
    """Whole-flat-space inputs (one fp32 gradient), for the unsharded comparison: dict(master, grad)."""
    rng = np.random.default_rng(w.seed)
    master = master_shard(w, 0, padded_n, rng)
    grad = rng.standard_normal(padded_n, dtype=np.float32) * np.float32(w.rep_std)
    grad[w.n:] = 0.0
    return {"master": master, "grad": grad}
