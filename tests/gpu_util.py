"""Helpers for the GPU parity tests: numpy <-> device tensors by bit pattern."""

import numpy as np
import torch

from bitcmp import assert_bits_equal, assert_bits_equal_nan, is_nan_bits  # noqa: F401 (re-exported)

DEV = "cuda:0"
_T16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def dev_rep(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Replica bits (uint16 for bf16/f16, float32 for f32) -> device tensor of that dtype."""
    if dtype == "f32":
        return dev_f32(a)
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV).view(_T16[dtype])


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def empty16(n: int, dtype: str, fill: float = 0.0) -> torch.Tensor:
    return torch.full((n,), fill, dtype=_T16[dtype], device=DEV)


def banner(msg: str):
    print(f"[gpu] {msg}", flush=True)

