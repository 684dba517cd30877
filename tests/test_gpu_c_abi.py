"""The fused step driven from plain C through include/zero_shard.h (no Python, no torch): on device
buffers, zero_adam_shard_step equals zero_reduce_shard followed by zero_host_adam_step, bit for bit;
the clipped path enqueued with nothing read back (squared norm, zero_clip_scale,
zero_adam_shard_step_dev_scale) gives C's own double evaluation of the clip rule and the host
update's bits, and so does the same update with t on the device (zero_adam_shard_step_dev_t),
which advances the counter, and the reduce pass with no workspace (zero_reduce_shard_static) equals
the one with a caller's partials; the offloaded step (zero_offload_step with the caller's pinned
staging and events) equals the fused step with either staging, and refuses pageable memory for
direct staging; the ZeRO-3 gather of a range across shards equals their concatenation; and the
fused step in an arena (zero_arena_layout, zero_arena_alloc) equals it on separate allocations
(tests/capi/step_check.c). The reduce pass and the host update are each pinned to
the oracle by the other tests."""

import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "zero_partition_plan_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fused_step_from_c(tmp_path):
    exe = tmp_path / "step_check"
    build = subprocess.run(
        ["gcc", "-std=gnu11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "capi", "step_check.c"), "-o", str(exe),
         "-L", LIBDIR, "-l:libzero_shard.so", f"-Wl,-rpath,{LIBDIR}",
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
         "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    print("[gpu] C ABI fused step check", flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "0 of 100003 elements differ" in run.stdout
