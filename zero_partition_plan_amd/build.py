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
SOURCES = [os.path.join(CSRC, "zero_host.cpp"), os.path.join(CSRC, "zero_step.hip"),
           os.path.join(CSRC, "zero_gather.hip"), os.path.join(CSRC, "zero_host_adam.cpp"),
           os.path.join(CSRC, "zero_offload.cpp"), os.path.join(CSRC, "zero_arena.cpp")]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
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


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the library to ``out`` (atomically replaced) and return its path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [f"-D{d}" for d in (defines or [])]
    cmd += ["-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args(argv)
    print(build(args.out, args.defines, verbose=True))


if __name__ == "__main__":
    main()
