"""The benchmark's measurement kernels (libzero_ceiling.so) with their factors at zero, as the
benchmark calls them on live state: the traffic twin leaves master, m, v unchanged and writes the
slot as the truncated bf16 of the master copy; the triad leaves its arrays unchanged. A refused
argument set launches nothing."""

import ctypes

import numpy as np
import pytest
import torch

import bench
from gpu_util import DEV, banner, bits16, bits32

pytestmark = pytest.mark.gpu


def test_twin_and_triad_leave_finite_state_unchanged():
    n = 256 * 37
    rng = np.random.default_rng(3)
    banner("ceiling kernels on live-like state")
    L = bench.ceiling_lib()
    reps = [torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).to(DEV).to(torch.bfloat16)
            for _ in range(8)]
    p, m, v = (torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(DEV) for _ in range(3))
    v = v.abs()
    slot = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    before = [bits32(x) for x in (p, m, v)]
    ptrs = (ctypes.c_void_p * 8)(*[r.data_ptr() for r in reps])
    stream = torch.cuda.current_stream().cuda_stream
    assert L.zero_ceiling_twin(ptrs, 8, n, p.data_ptr(), m.data_ptr(), v.data_ptr(), slot.data_ptr(),
                               0.0, stream) == 0
    assert L.zero_ceiling_triad(p.data_ptr(), m.data_ptr(), n, 0.0, stream) == 0
    torch.cuda.synchronize()
    for a, b in zip((p, m, v), before):
        assert np.array_equal(bits32(a), b)
    assert np.array_equal(bits16(slot), (before[0] >> 16).astype(np.uint16))
    # arguments the kernels do not take: a size off the 256-element tile, a replica count of 7
    assert L.zero_ceiling_twin(ptrs, 8, n - 1, p.data_ptr(), m.data_ptr(), v.data_ptr(), slot.data_ptr(),
                               0.0, stream) == 1
    assert L.zero_ceiling_twin(ptrs, 7, n, p.data_ptr(), m.data_ptr(), v.data_ptr(), slot.data_ptr(),
                               0.0, stream) == 1
    assert L.zero_ceiling_triad(p.data_ptr(), m.data_ptr(), n + 3, 0.0, stream) == 1
