"""Model parameter lists and the five synthetic workloads.

Flattening reading: tensors are concatenated in the order listed, row-major, with no per-tensor
padding. Init kinds: "normal" (matrices and embeddings, N(0, 0.02) with 0.02 the standard
deviation), "one" (norm weights), "zero" (biases).

  gpt2-small : token embedding 50257x768, positions 1024x768, 12 blocks of (ln_1 w/b, qkv 768x2304,
               proj 768x768, ln_2 w/b, fc 768x3072, fc_proj 3072x768), ln_f w/b; no linear biases,
               output head tied to the token embedding -> 124,356,864
  llama-7b   : embed 32000x4096, 32 blocks of (attn norm, q/k/v/o 4096x4096, mlp norm, gate and up
               4096x11008, down 11008x4096), final norm, untied head 32000x4096 -> 6,738,415,616
  llama-13b  : same with d 5120, ffn 13824, 40 blocks, vocab 32000 -> 13,015,864,320
  gpt3-175b  : wte 50257x12288, wpe 2048x12288, 96 blocks of (ln_1 w/b, qkv 12288x36864 + bias,
               proj 12288x12288 + bias, ln_2 w/b, fc 12288x49152 + bias, fc2 49152x12288 + bias),
               ln_f w/b -> 174,604,259,328
"""

from __future__ import annotations

from dataclasses import dataclass, field
from functools import lru_cache


def _gpt2_small():
    d, v, ctx, L = 768, 50257, 1024, 12
    out = [("wte", v * d, "normal"), ("wpe", ctx * d, "normal")]
    for i in range(L):
        out += [
            (f"h{i}.ln_1.w", d, "one"), (f"h{i}.ln_1.b", d, "zero"),
            (f"h{i}.attn.qkv", d * 3 * d, "normal"), (f"h{i}.attn.proj", d * d, "normal"),
            (f"h{i}.ln_2.w", d, "one"), (f"h{i}.ln_2.b", d, "zero"),
            (f"h{i}.mlp.fc", d * 4 * d, "normal"), (f"h{i}.mlp.proj", 4 * d * d, "normal"),
        ]
    out += [("ln_f.w", d, "one"), ("ln_f.b", d, "zero")]
    return out


def _llama(d, ffn, L, vocab):
    out = [("embed", vocab * d, "normal")]
    for i in range(L):
        out += [(f"l{i}.attn_norm", d, "one")]
        out += [(f"l{i}.{w}", d * d, "normal") for w in ("q", "k", "v", "o")]
        out += [(f"l{i}.mlp_norm", d, "one")]
        out += [(f"l{i}.gate", d * ffn, "normal"), (f"l{i}.up", d * ffn, "normal"),
                (f"l{i}.down", ffn * d, "normal")]
    out += [("norm", d, "one"), ("lm_head", vocab * d, "normal")]
    return out


def _gpt3_175b():
    d, v, ctx, L = 12288, 50257, 2048, 96
    out = [("wte", v * d, "normal"), ("wpe", ctx * d, "normal")]
    for i in range(L):
        out += [
            (f"h{i}.ln_1.w", d, "one"), (f"h{i}.ln_1.b", d, "zero"),
            (f"h{i}.attn.qkv", d * 3 * d, "normal"), (f"h{i}.attn.qkv.b", 3 * d, "zero"),
            (f"h{i}.attn.proj", d * d, "normal"), (f"h{i}.attn.proj.b", d, "zero"),
            (f"h{i}.ln_2.w", d, "one"), (f"h{i}.ln_2.b", d, "zero"),
            (f"h{i}.mlp.fc", d * 4 * d, "normal"), (f"h{i}.mlp.fc.b", 4 * d, "zero"),
            (f"h{i}.mlp.proj", 4 * d * d, "normal"), (f"h{i}.mlp.proj.b", d, "zero"),
        ]
    out += [("ln_f.w", d, "one"), ("ln_f.b", d, "zero")]
    return out


MODELS = {
    "gpt2-small": _gpt2_small,
    "llama-7b": lambda: _llama(4096, 11008, 32, 32000),
    "llama-13b": lambda: _llama(5120, 13824, 40, 32000),
    "gpt3-175b": _gpt3_175b,
}


@lru_cache(maxsize=None)
def param_list(model: str) -> tuple:
    """((name, numel, init_kind), ...) in flattening order."""
    return tuple(MODELS[model]())


@lru_cache(maxsize=None)
def flat_count(model: str) -> int:
    return sum(n for _, n, _ in param_list(model))


def _layer_key(name: str) -> str:
    head = name.split(".")[0]
    if head[0] in "hl" and head[1:].isdigit():
        return head                          # a transformer block
    return "embed" if head in ("wte", "wpe", "embed") else "final"


@lru_cache(maxsize=None)
def layer_ranges(model: str) -> tuple:
    """((layer, start, end), ...): consecutive flat ranges of the embeddings, each block, and the
    final norm / head, in flattening order (the unit a ZeRO-3 forward gathers at a time)."""
    out = []
    pos = 0
    for name, n, _ in param_list(model):
        key = _layer_key(name)
        if out and out[-1][0] == key:
            out[-1] = (key, out[-1][1], pos + n)
        else:
            out.append((key, pos, pos + n))
        pos += n
    return tuple(out)


@lru_cache(maxsize=None)
def init_ranges(model: str) -> tuple:
    """((start, end, kind), ...) over the flat space, only the non-"normal" ranges, merged."""
    out = []
    pos = 0
    for _, n, kind in param_list(model):
        if kind != "normal":
            if out and out[-1][2] == kind and out[-1][1] == pos:
                out[-1] = (out[-1][0], pos + n, kind)
            else:
                out.append((pos, pos + n, kind))
        pos += n
    return tuple(out)


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the per-rank step (sizes, distributions, seed)."""
    name: str
    model: str | None          # None: an unstructured flat space of ``n`` elements
    n: int
    nd: int
    ranks: tuple               # ranks stepped
    reps: int                  # gradient replicas summed (R)
    rep_dtype: str             # "f32" | "f16" | "bf16"
    rep_std: float             # replica draw: N(0, rep_std) (times loss_scale for f16)
    master_std: float = 0.02
    loss_scale: float = 1.0    # replicas hold grad * loss_scale
    inf_rate: float = 0.0      # per replica element, +inf injected with this probability
    max_norm: float | None = None
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    wd_mode: str = "adamw"
    warm_steps: int = 0        # state drawn as if this many steps had run; first step t = warm+1
    steps: int = 1             # steps in a parity run
    out_dtypes: tuple = ("bf16",)
    seed: int = 0
    window: int | None = None  # replicas hold one window of this many elements, re-read per window
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", model=None, n=1_000_003, nd=4, ranks=(0, 1, 2, 3), reps=1, rep_dtype="f32",
        rep_std=1e-3, weight_decay=0.0, steps=3, out_dtypes=("bf16", "f16"), seed=0,
        notes="odd N forces one element of padding; one fp32 gradient reused for all 3 steps"),
    "gpt2": Workload(
        name="gpt2", model="gpt2-small", n=flat_count("gpt2-small"), nd=8, ranks=(3,), reps=8,
        rep_dtype="bf16", rep_std=1e-3, weight_decay=0.01, steps=2, seed=1),
    "llama7b": Workload(
        name="llama7b", model="llama-7b", n=flat_count("llama-7b"), nd=8, ranks=(0,), reps=8,
        rep_dtype="bf16", rep_std=1e-4, weight_decay=0.01, warm_steps=10, steps=1, seed=2),
    "llama13b": Workload(
        name="llama13b", model="llama-13b", n=flat_count("llama-13b"), nd=16, ranks=(5,), reps=16,
        rep_dtype="f16", rep_std=1e-4, loss_scale=65536.0, inf_rate=1e-4, max_norm=1.0,
        weight_decay=0.01, steps=1, out_dtypes=("f16",), seed=3),
    "gpt3": Workload(
        name="gpt3", model="gpt3-175b", n=flat_count("gpt3-175b"), nd=64, ranks=(0,), reps=64,
        rep_dtype="bf16", rep_std=1e-4, weight_decay=0.1, steps=1, seed=4, window=64 << 20),
}
