"""torch generators that draw the large workloads directly in device memory.

Same recipe as ``workloads.host`` (master, replicas 0..R-1 with any injected +inf, then warm m, v),
drawn with a seeded ``torch.Generator`` on the device (Philox), so a multi-GB shard never crosses
PCIe. 16-bit replicas are torch's conversions of fp32 draws. Replicas are one [R, size] tensor (one
allocation, rows contiguous), or a list of R row tensors when the caller supplies the storage.
"""

from __future__ import annotations

import math

import torch

from .shapes import Workload, init_ranges

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _new(empty, name: str, size: int, dtype, device) -> torch.Tensor:
    if empty is None:
        return torch.empty(size, dtype=dtype, device=device)
    t = empty(name, size, dtype)
    if t.shape != (size,) or t.dtype != dtype:
        raise ValueError(f"storage for {name}: got {tuple(t.shape)} {t.dtype}, need ({size},) {dtype}")
    return t


def master_shard(w: Workload, begin: int, size: int, gen, device, empty=None) -> torch.Tensor:
    x = _new(empty, "master", size, torch.float32, device)
    torch.randn(size, generator=gen, out=x)
    x.mul_(w.master_std)
    if w.model is not None:
        end = begin + size
        for s, e, kind in init_ranges(w.model):
            lo, hi = max(s, begin), min(e, end)
            if lo < hi:
                x[lo - begin:hi - begin].fill_(1.0 if kind == "one" else 0.0)
    if begin + size > w.n:
        x[max(0, w.n - begin):].zero_()
    return x


def replicas(w: Workload, size: int, valid: int, gen, device, reps: int | None = None, empty=None):
    r = w.reps if reps is None else reps
    if empty is None:
        out = torch.empty((r, size), dtype=_DT[w.rep_dtype], device=device)
    else:
        out = [_new(empty, f"rep{k}", size, _DT[w.rep_dtype], device) for k in range(r)]
    for k in range(r):
        x = torch.randn(size, generator=gen, device=device, dtype=torch.float32)
        x.mul_(w.rep_std * (w.loss_scale if w.rep_dtype == "f16" else 1.0))
        if valid < size:
            x[valid:].zero_()
        out[k].copy_(x)
        del x
    if w.inf_rate > 0.0:
        for k in range(r):
            mask = torch.rand(size, generator=gen, device=device) < w.inf_rate
            if valid < size:
                mask[valid:] = False
            out[k].masked_fill_(mask, float("inf"))
            del mask
    return out


def warm_state(w: Workload, size: int, valid: int, gen, device, empty=None):
    m = _new(empty, "m", size, torch.float32, device).zero_()
    v = _new(empty, "v", size, torch.float32, device).zero_()
    k = w.warm_steps
    if k > 0:
        sg = w.rep_std * math.sqrt(w.reps)
        sm = sg * (1 - w.beta1) * math.sqrt((1 - w.beta1 ** (2 * k)) / (1 - w.beta1 ** 2))
        m.normal_(0.0, sm, generator=gen)
        v.uniform_(0.5, 1.5, generator=gen).mul_((1 - w.beta2 ** k) * sg * sg)
        if valid < size:
            m[valid:].zero_()
            v[valid:].zero_()
    return m, v


def rank_inputs(w: Workload, begin: int, size: int, valid: int, device="cuda",
                seed_offset: int = 0, rep_size: int | None = None, empty=None):
    """dict(master, m, v, reps); ``rep_size`` < size draws one replica window (re-read per window).

    ``empty(name, numel, dtype)``, when given, supplies each array's storage (names master, m, v,
    rep0 .. rep{R-1}), for example views of one arena; the values drawn are the same either way.
    """
    gen = generator(w.seed + seed_offset, device)
    master = master_shard(w, begin, size, gen, device, empty)
    rs = size if rep_size is None else rep_size
    reps = replicas(w, rs, min(valid, rs), gen, device, empty=empty)
    m, v = warm_state(w, size, valid, gen, device, empty)
    return {"master": master, "m": m, "v": v, "reps": reps}
