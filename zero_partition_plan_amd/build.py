"""Compile libzero_shard.so in-tree with hipcc for gfx950.

    python -m zero_partition_plan_amd.build [-D NAME=VALUE ...] [--out PATH]

Flags that matter for the numerics: -ffp-contract=off (no fused multiply-add, so every fp32
operation is rounded on its own) and correctly rounded fp32 division and square root. Packed fp32
instructions are disabled (-packed-fp32-ops) for all device code.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzero_shard.so")
# the benchmark's measurement kernels (traffic twin, triad): a library of their own, not the step's
CEILING_LIB = os.path.join(PKG, "libzero_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "zero_ceiling.hip")]
SOURCES = [os.path.join(CSRC, "zero_host.cpp"), os.path.join(CSRC, "zero_step.hip"),
           os.path.join(CSRC, "zero_gather.hip"), os.path.join(CSRC, "zero_host_adam.cpp"),
           os.path.join(CSRC, "zero_offload.cpp"), os.path.join(CSRC, "zero_arena.cpp")]
# the step's kernel variants, compiled once per replica / output dtype pair (zero_dtype values:
# 0 fp32, 1 fp16, 2 bf16; an fp32 "output" means none and also carries the reduce pass)
STEP_KERNELS = os.path.join(CSRC, "zero_step_kernels.hip")
STEP_PAIRS = [(r, o) for r in (0, 1, 2) for o in (0, 1, 2)]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-fno-math-errno",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _units():
    """(source, extra defines, object stem) for every object of the library."""
    units = [(src, [], os.path.splitext(os.path.basename(src))[0]) for src in SOURCES]
    units += [(STEP_KERNELS, [f"ZERO_STEP_RDT={r}", f"ZERO_STEP_ODT={o}"], f"zero_step_kernels_{r}{o}")
              for r, o in STEP_PAIRS]
    return units


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False,
          jobs: int | None = None, ceiling_out: str | None = CEILING_LIB) -> str:
    """Compile the library to ``out`` (atomically replaced) and return its path; with
    ``ceiling_out``, also the measurement library there. The objects build in parallel (``jobs``
    processes, default: the CPU count, at most 16) in a scratch directory."""
    import concurrent.futures
    import tempfile
    base = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    base += [f"-D{d}" for d in (defines or [])]
    jobs = jobs or min(16, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="zero_build_") as tmpdir:
        cmds, objs, ceil_objs = [], [], []
        units = [(u, objs) for u in _units()]
        if ceiling_out:
            units += [((src, [], "ceil_" + os.path.splitext(os.path.basename(src))[0]), ceil_objs)
                      for src in CEILING_SOURCES]
        for (src, defs, stem), dest in units:
            obj = os.path.join(tmpdir, stem + ".o")
            cmds.append([*base, "-c", *[f"-D{d}" for d in defs], "-o", obj, src])
            dest.append(obj)
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        links = [(out, objs)] + ([(ceiling_out, ceil_objs)] if ceiling_out else [])
        for dst, os_ in links:
            _run([hipcc(), *FLAGS, "-shared", "-o", dst + ".tmp", *os_], verbose)
        for dst, _ in links:
            os.replace(dst + ".tmp", dst)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measurement library")
    args = ap.parse_args(argv)
    print(build(args.out, args.defines, verbose=True, ceiling_out=None if args.no_ceiling else CEILING_LIB))


if __name__ == "__main__":
    main()
