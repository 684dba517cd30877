"""The C ABI from plain C: include/zero_shard.h compiles as pedantic C99 and the host entry points,
called from C, give the oracle's partition plan, shard ranges, per-stage bytes held and sent, and
the fp32 Adam constants the oracle derives."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "zero_partition_plan_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_host_entry_points_from_c99(tmp_path):
    exe = tmp_path / "host_check"
    build = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "capi", "host_check.c"), "-o", str(exe), "-L", LIBDIR,
         "-l:libzero_shard.so", f"-Wl,-rpath,{LIBDIR}"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr[-3000:]
    seen = {"plan": 0, "range": 0, "stage": 0, "comm": 0}
    for line in run.stdout.splitlines():
        kind, rest = line.split(" ", 1)
        if kind in ("plan", "range", "stage", "comm"):
            lhs, rhs = rest.split(" -> ")
            a = [int(x) for x in lhs.split()]
            got = [int(x) for x in rhs.split()]
            plan = O.partition_plan(a[0], a[1], a[2])
            if kind == "plan":
                assert got == [plan.shard_elems, plan.padded_n, plan.pad], line
            elif kind == "range":
                assert got == list(O.shard_range(plan, a[3])), line
            elif kind == "comm":
                assert got == list(O.stage_comm_bytes(plan, a[3], 2, 2)), line
            else:
                want = O.stage_bytes_exact(plan, a[3], 2, 2, 12)
                assert got == [int(x) for x in want], line
            seen[kind] += 1
        elif kind == "scalars":
            sc = O.adam_scalars(O.AdamHParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                              weight_decay=0.01, step=11))
            got = [np.float32(float.fromhex(x)) for x in rest.split()]
            want = [sc.b1, sc.b2, sc.c1, sc.c2, sc.ss, sc.bc, sc.e, sc.dec, sc.w]
            assert [g.view(np.uint32) for g in got] == [np.float32(w).view(np.uint32) for w in want]
        elif kind == "arena":
            offs = [int(x) for x in rest.split()]
            q = 4 << 20                                   # granule of arrays this small
            assert offs[0] % q == 0 and (offs[1] + 400) % q == 2048 and offs[2] % q == 0
            assert offs[1] >= offs[0] + 1000 and offs[2] >= offs[1] + 4000 and offs[3] == offs[2] + 4000
        elif kind == "status":
            assert rest
    assert seen == {"plan": 4, "range": 4 + 8 + 8 + 16, "stage": 16, "comm": 16}
