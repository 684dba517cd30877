#!/usr/bin/env python3
"""Throughput of one data-parallel rank's sharded AdamW step on one MI355X.

Default workload: the Llama-7B-shaped flat parameter space (6,738,415,616 elements) over Nd = 8
ranks, one rank's 842,301,952-element shard: 8 bf16 gradient replicas summed in fixed order,
AdamW on the fp32 master / m / v (warm state, t = 11), bf16 cast into the rank's slot of the full
gathered parameter buffer. One step = one fused kernel launch. Inputs are drawn on the device and
are resident in HBM before the timed region, all arrays of the step in one arena laid out by
zero_arena_layout (arrays a kernel walks together start at staggered offsets past 256 MiB lines).

Prints one JSON line (see the fields below). Flags:
  --gpus N         only 1 is supported: this path runs on one GPU's shard
  --steps K        timed steps (default: per workload, a timed region of a few seconds, e.g.
                   1000 for llama7b)
  --warmup W       untimed steps first (default 3)
  --config C       the same by config number: 2 gpt2, 3 llama7b, 4 llama13b, 5 gpt3
  --workload NAME  llama7b (default), gpt2, llama13b (two-pass clip path), gpt3 (64 Mi windows),
                   gather7b (ZeRO-3: every Llama-7B layer gathered from its 8 rank shards),
                   offload7b (ZeRO-Offload: the 7B shard's Adam state in host memory)
  --placement P    arena (default) or separate: every array of the step in its own allocation
  --no-context     skip the context legs (copy ceiling, separate-placement step, cold launches, graph
                   replay, the offloaded step's direct-staging legs)
  --offload-staging copy|direct  offload7b: gradient chunks copied from device staging (default) or
                   written into pinned host memory by the reduce kernel
  --cpu-seconds S  budget of the oracle's CPU baseline (default 12; 0 skips it)
  --copy-calib MB  also run a plain device copy of MB MiB 5 times (for counter calibration)
  --summarize      (no GPU) turn the rocprofv3 CSVs of the profile commands into the summaries
                   under profiles/ and exit
  --profile-commands  print the three rocprofv3 commands for --workload, and the same bench
                   command untraced, and exit

The kernel-trace summary and the two counter passes (FETCH_SIZE, then WRITE_SIZE) are taken by the
commands --profile-commands prints; their CSVs land in <root>/prof_<workload>_{trace,fetch,write}
and their console output in the .log file of the same name, where <root> is $ZERO_PROFILE_ROOT
(default profile_runs, relative to the repository root). The untraced run (prof_<workload>_plain.log)
gives the event figure without the profiler's per-dispatch cost, for comparison in the summary.
"""

from __future__ import annotations

import argparse
import dataclasses
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sharded Adam step params/s per GPU + achieved HBM GB/s vs peak (7B, Nd=8)"
HBM_PEAK_GBS = 8000.0
_CSRC = os.path.join(ROOT, "zero_partition_plan_amd", "csrc")
# the device sources each kernel is built from
KERNEL_SRCS = {k: [os.path.join(_CSRC, f) for f in fs] for k, fs in {
    "k_adam_step": ("zero_step_kernels.hip", "zero_step.h", "zero_device.h"),
    "k_reduce": ("zero_step_kernels.hip", "zero_step.h", "zero_device.h"),
    "k_gather": ("zero_gather.hip", "zero_device.h"),
}.items()}
PROFILES = os.path.join(ROOT, "profiles")
CALIB_MIB = 1024

WL_DESC = {
    "llama7b": "Llama-7B-shaped flat space (6,738,415,616 params), Nd=8, rank 0 shard, "
               "8 bf16 replicas, warm AdamW state",
    "gpt2": "GPT-2-small-shaped flat space (124,356,864 params), Nd=8, rank 3 shard, 8 bf16 replicas",
    "llama13b": "Llama-13B-shaped flat space (13,015,864,320 params), Nd=16, rank 5 shard, "
                "16 fp16 replicas x 2^16 with 0.01% +inf (every step overflows and is skipped), "
                "two-pass clip path",
    "llama13b-clean": "Llama-13B-shaped flat space (13,015,864,320 params), Nd=16, rank 5 shard, "
                      "16 fp16 replicas x 2^16, no overflow, two-pass clip path",
    "gpt3": "GPT-3-175B-shaped flat space (174,604,259,328 params), Nd=64, rank 0 shard, "
            "64 bf16 replicas per 64 Mi window",
    "gather7b": "ZeRO-3 parameter gather: the 34 layers of the Llama-7B-shaped bf16 parameters "
                "(6,738,415,616) rebuilt in turn from 8 rank shards",
    "offload7b": "ZeRO-Offload: Llama-7B-shaped shard (842,301,952 params, Nd=8, rank 0), 8 bf16 "
                 "replicas summed on the GPU, AdamW on fp32 state in host memory, bf16 back to the slot",
}
GATHER_LAYERS = 34          # embeddings, 32 blocks, final norm + head
OFFLOAD_CHUNK = 32 << 20    # elements per pipeline chunk
OFFLOAD_THREADS = 16        # host threads: a 16-core host share per GPU
# default timed steps per workload: about 5 s of timed work each
DEFAULT_STEPS = {"llama7b": 1000, "gpt2": 10000, "llama13b": 500, "llama13b-clean": 500, "gpt3": 60,
                 "gather7b": 300, "offload7b": 30}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_only(text: str) -> str:
    """C/C++ source with its comments removed and every run of whitespace made one space; string
    and character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash(kernel: str) -> str:
    """sha256[:16] over the code (comments and layout left out) of the device sources of
    ``kernel``: a counter summary is used only for the exact code it was taken on."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS[kernel]:
        h.update(code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- bytes

def _rb(w) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[w.rep_dtype]


def dominant_kernels(workload: str) -> list:
    """Library kernels of one step, the one that moves the most bytes first."""
    if workload == "gather7b":
        return ["k_gather"]
    if workload == "offload7b":
        return ["k_reduce"]
    return ["k_reduce", "k_adam_step"] if workload.startswith("llama13b") else ["k_adam_step"]


def kernel_bytes_per_elem(workload: str) -> dict:
    """Algorithmic HBM bytes each library kernel must move per shard element."""
    from workloads import WORKLOADS
    if workload == "gather7b":
        return {"k_gather": 2 + 2}            # each bf16 parameter read from its shard and written
    if workload == "offload7b":
        return {"k_reduce": 8 * 2 + 4}        # 8 bf16 replicas in, the fp32 gradient chunk out
    w = WORKLOADS["llama13b" if workload.startswith("llama13b") else workload]
    if workload.startswith("llama13b"):
        # pass 1 reads R replicas and writes the fp32 gradient; pass 2 reads it, reads and
        # writes master/m/v and writes the 16-bit parameters
        return {"k_reduce": w.reps * _rb(w) + 4, "k_adam_step": 4 + 24 + 2}
    return {"k_adam_step": w.reps * _rb(w) + 24 + 2}


def shard_elems(w) -> int:
    per = -(-w.n // w.nd)
    return per


def launch_elems(workload: str) -> float:
    """Shard elements one launch of the dominant kernel covers, as the mean over one step's launches
    (the layer gather's layers differ in size, and a windowed shard ends in a shorter window), so
    that bytes per element x this / the mean launch time is the step's algorithmic bytes over its
    total kernel time."""
    from workloads import WORKLOADS
    if workload == "gather7b":
        return WORKLOADS["llama7b"].n / GATHER_LAYERS
    if workload == "offload7b":         # the step's chunks: 25 of 32 Mi and a shorter last one
        S = shard_elems(WORKLOADS["llama7b"])
        return S / -(-S // OFFLOAD_CHUNK)
    w = WORKLOADS["llama13b" if workload.startswith("llama13b") else workload]
    S = shard_elems(w)
    return S / -(-S // (w.window or S))


def launches_per_step(workload: str) -> int:
    """Library calls one step makes (timed spans), for reserving their events up front."""
    from workloads import WORKLOADS
    if workload == "gather7b":
        return GATHER_LAYERS
    if workload == "offload7b":
        return 1
    w = WORKLOADS["llama13b" if workload.startswith("llama13b") else workload]
    S = shard_elems(w)
    return 2 if workload.startswith("llama13b") else -(-S // (w.window or S))


def algorithmic_bytes_per_launch(workload: str) -> float:
    k = dominant_kernels(workload)[0]
    return float(kernel_bytes_per_elem(workload)[k]) * launch_elems(workload)


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash(kernel):
        return None
    return float(m_bytes.group(1))


# ----------------------------------------------------------------------------- profiles

def profile_root() -> str:
    """Where the profiling commands write their output ($ZERO_PROFILE_ROOT, default profile_runs)."""
    return os.environ.get("ZERO_PROFILE_ROOT", "profile_runs")


def profile_dirs(workload: str) -> dict:
    return {k: os.path.join(profile_root(), f"prof_{workload}_{k}")
            for k in ("trace", "fetch", "write", "plain")}


def profile_commands(workload: str) -> dict:
    d = profile_dirs(workload)
    run = f"python -u bench.py --workload {workload} --no-context"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats -T -d {d['trace']} -o kt -f csv -- "
                 f"{run} --steps 10 --warmup 2 --cpu-seconds 0",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -T -d {d['fetch']} -o pmc -f csv -- "
                 f"{run} --steps 3 --warmup 1 --cpu-seconds 0 --copy-calib {CALIB_MIB}",
        "write": f"rocprofv3 --pmc WRITE_SIZE -T -d {d['write']} -o pmc -f csv -- "
                 f"{run} --steps 3 --warmup 1 --cpu-seconds 0 --copy-calib {CALIB_MIB}",
        "plain": f"{run} --steps 10 --warmup 2 --cpu-seconds 0",
    }


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _agent(dirpath):
    for r in _csv(_find(dirpath, "_agent_info.csv")):
        if r.get("Agent_Type") == "GPU":
            return f"{r.get('Name')} ({r.get('Cu_Count')} CUs, {r.get('Num_Xcc')} XCDs)"
    return "unknown"


def _logged(dirpath, pattern):
    log_path = dirpath + ".log"
    if os.path.exists(log_path):
        m = re.search(pattern, open(log_path).read())
        if m:
            return m.group(1)
    return None


def summarize(workload: str):
    """Write profiles/<kernel>_<workload>_trace.md and _counters.md from the profile CSVs."""
    kernels = dominant_kernels(workload)
    cmds, dirs = profile_commands(workload), profile_dirs(workload)
    os.makedirs(PROFILES, exist_ok=True)
    n_launch = launch_elems(workload)
    bpe = kernel_bytes_per_elem(workload)

    stats = _csv(_find(dirs["trace"], "_kernel_stats.csv"))
    src_hash = _logged(dirs["trace"], r"kernel source sha256\[:16\] ([0-9a-f]{16})")
    lines = [f"# {kernels[0]} kernel trace, {workload} shard", "",
             f"- command (repo root): `{cmds['trace']}`",
             f"- GPU: {_agent(dirs['trace'])}",
             f"- kernel source sha256[:16]: `{src_hash}`",
             f"- workload: {WL_DESC[workload]}; {n_launch:,.0f} shard elements per launch (mean over "
             f"a step's launches)", "",
             "| kernel | calls | avg ms | min ms | max ms | share | algorithmic GB/s at avg |",
             "|---|---|---|---|---|---|---|"]
    for r in stats:
        name, avg = r["Name"], float(r["AverageNs"])
        gbs = f"{bpe[name] * n_launch / avg:.0f}" if name in bpe else "-"
        if workload == "llama13b" and name == "k_adam_step":
            gbs = "- (skip flag set: every block exits at once)"
        lines.append(f"| {name} | {r['Calls']} | {avg / 1e6:.4f} | {float(r['MinNs']) / 1e6:.4f} | "
                     f"{float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.1f}% | {gbs} |")
    bench_line = _logged(dirs["trace"], r"(\{\"metric\".*\})")
    if bench_line:
        rl = json.loads(bench_line)["roofline"]
        lines += ["", f"bench.py's own HIP-event figure in the same run: {rl['avg_launch_ms']:.4f} ms "
                      f"per launch of {rl['kernel']} ({rl['achieved']:.0f} GB/s algorithmic)."]
    plain_line = _logged(dirs["plain"], r"(\{\"metric\".*\})")
    if plain_line:
        rl = json.loads(plain_line)["roofline"]
        lines += [f"The same bench command without the profiler (`{cmds['plain']}`): "
                  f"{rl['avg_launch_ms']:.4f} ms per launch ({rl['achieved']:.0f} GB/s algorithmic)."]
    lines += ["", "Kernels other than the library's are the seeded input generators (torch) that run "
              "before the timed region."]
    out = os.path.join(PROFILES, f"{kernels[0]}_{workload}_trace.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("wrote", out)

    per, calib = {}, {}
    for c in ("fetch", "write"):
        rows = _csv(_find(dirs[c], "_counter_collection.csv"))
        per[c] = {}
        for k in kernels:
            vals = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == k]
            per[c][k] = sum(vals) / len(vals) if vals else None
        # the calibration copies are the run's last CALIB_MIB-sized device copies
        big = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
               and float(r["Counter_Value"]) > 0.25 * CALIB_MIB * 1024]
        calib[c] = sum(big[-5:]) / len(big[-5:])
    f_fetch = CALIB_MIB * 1024 / calib["fetch"]
    f_write = CALIB_MIB * 1024 / calib["write"]
    src_hash = _logged(dirs["fetch"], r"kernel source sha256\[:16\] ([0-9a-f]{16})")
    lines = [f"# {', '.join(kernels)} HBM traffic counters, {workload} shard", "",
             f"- FETCH_SIZE pass (repo root): `{cmds['fetch']}`",
             f"- WRITE_SIZE pass (repo root): `{cmds['write']}`",
             f"- GPU: {_agent(dirs['fetch'])}",
             f"- kernel source sha256[:16]: `{src_hash}`",
             f"- calibration: a plain device copy of {CALIB_MIB} MiB (torch copy_, "
             f"__amd_rocclr_copyBuffer) reads FETCH_SIZE {calib['fetch']:.1f} KiB and writes "
             f"WRITE_SIZE {calib['write']:.1f} KiB per dispatch for {CALIB_MIB * 1024} KiB each way, "
             f"so HBM bytes = FETCH_SIZE x {f_fetch:.4f} KiB + WRITE_SIZE x {f_write:.4f} KiB", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | read bytes | written bytes | "
             "calibrated / algorithmic |", "|---|---|---|---|---|---|"]
    dominant_total = None
    for k in kernels:
        fb, wb = per["fetch"][k], per["write"][k]
        if fb is None or wb is None:
            lines.append(f"| {k} | - | - | - | - | - |")
            continue
        rb, wrb = fb * f_fetch * 1024, wb * f_write * 1024
        ratio = f"{(rb + wrb) / (bpe[k] * n_launch):.4f}"
        if workload == "llama13b" and k == "k_adam_step":
            ratio = "- (skip flag set: every block exits at once)"
        lines.append(f"| {k} | {fb:.1f} | {wb:.1f} | {rb:,.0f} | {wrb:,.0f} | {ratio} |")
        if dominant_total is None:
            dominant_total = rb + wrb
    alg = algorithmic_bytes_per_launch(workload)
    lines += ["", f"Dominant kernel: {kernels[0]}",
              f"HBM bytes per launch (calibrated): {dominant_total:.6e}",
              f"Algorithmic bytes per launch: {alg:.6e} ({bpe[kernels[0]]} B per shard element)"]
    out = os.path.join(PROFILES, f"{kernels[0]}_{workload}_counters.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("wrote", out)


# ----------------------------------------------------------------------------- workloads

def setup(name: str, placement: str = "arena"):
    """Inputs of one rank's step, drawn on the device. With ``placement`` "arena" every array of the
    step lives in one allocation laid out by zero_arena_layout; "separate" gives each its own."""
    import torch

    import zero_partition_plan_amd as Z
    from workloads import WORKLOADS
    from workloads import device as D
    from workloads.placement import step_arrays

    w = WORKLOADS["llama13b"] if name.startswith("llama13b") else WORKLOADS[name]
    if name == "llama13b-clean":
        w = dataclasses.replace(w, inf_rate=0.0)
    two_pass = name.startswith("llama13b")
    plan = Z.zero_partition_plan(w.n, w.nd)
    rank = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, rank)
    S = plan.shard_elems
    dev = torch.device("cuda:0")
    log(f"workload {name}: N={w.n} Nd={w.nd} rank={rank} S={S} R={w.reps}x{w.rep_dtype} "
        f"placement={placement}")
    storage, views = None, None
    if placement == "arena":
        storage, views = Z.arena(step_arrays(w, S, begin, plan.padded_n, two_pass), device=dev)
        log(f"arena: {storage.numel() / 2**30:.2f} GiB for {len(views)} arrays, "
            f"{'physically contiguous' if storage.zero_arena_contiguous else 'not contiguous'}")
        placement = "arena, contiguous" if storage.zero_arena_contiguous else "arena"
    empty = (lambda nm, n, dt: views[nm]) if views else None
    inp = D.rank_inputs(w, begin, S, valid, device=dev, rep_size=w.window, empty=empty)
    out_t = torch.float16 if w.out_dtypes[0] == "f16" else torch.bfloat16
    state = dict(w=w, plan=plan, S=S, begin=begin, inp=inp, t=w.warm_steps + 1, arena=storage,
                 placement=placement)
    if w.window is None and not two_pass:
        state["full"] = (views["full"].zero_() if views else
                         torch.zeros(plan.padded_n, dtype=out_t, device=dev))
        state["slot"] = state["full"][begin:begin + S]
    else:
        state["slot"] = views["slot"].zero_() if views else torch.zeros(S, dtype=out_t, device=dev)
    if two_pass:
        state["g"] = views["g"] if views else torch.empty(S, device=dev)
        state["flag"] = torch.zeros(1, dtype=torch.int32, device=dev)
        state["host_flag"] = torch.zeros(1, dtype=torch.int32, pin_memory=True)
        state["flag_ready"] = torch.cuda.Event()
        state["flag_pending"] = None       # Spans of the step whose flag the host has not read yet
        state["skipped"] = 0
        state["parts"] = torch.empty(Z.zero_sq_partials_len(S), dtype=torch.float64, device=dev)
        state["sq"] = torch.empty(1, dtype=torch.float64, device=dev)
        state["gs"] = torch.empty(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    return state


def placement_context(name: str, steps: int = 5):
    """The same step with every array in its own allocation (the default allocator's placement)."""
    import torch
    st = setup(name, "separate")
    step = step_two_pass if name.startswith("llama13b") else step_fused
    for _ in range(2):
        step(st, Spans(False))
    torch.cuda.synchronize()
    e0, e1 = new_event(True), new_event()
    for _ in range(steps):
        step(st, Spans(False))
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del st
    torch.cuda.empty_cache()
    return {"separate_ms_per_step": ms, "steps": steps,
            "note": "the same step with master, m, v, every replica row and the output each in its own "
                    "allocation; the timed line above places them in one arena (zero_arena_layout)"}


def _interleaved(legs, calls: int = 5, rounds: int = 3):
    """ms per call of each (name, fn) leg, timed in alternation (calls per leg per round, rounds
    rounds) so that drift on the box hits every leg alike; the median round of each."""
    import torch
    got = {name: [] for name, _ in legs}
    for _ in range(rounds):
        for name, fn in legs:
            fn()
            torch.cuda.synchronize()
            e0, e1 = new_event(True), new_event()
            for _ in range(calls):
                fn()
            e1.record()
            torch.cuda.synchronize()
            got[name].append(e0.elapsed_time(e1) / calls)
    return {name: pct(xs, 0.5) for name, xs in got.items()}


def odd_slot_context(st):
    """The 7B step with its slot one element past its place (2 bytes past a 4-byte word, as rank
    r's slot r*S of the gathered buffer is when S is odd: the word-realigning store path), against
    the aligned step, timed in alternation in the same arena."""
    import zero_partition_plan_amd as Z
    inp, S, b = st["inp"], st["S"], st["begin"]
    odd = Z.AdamStep(inp["reps"], S, inp["master"], inp["m"], inp["v"], out=st["full"][b + 1:b + 1 + S])

    def aligned():
        step_fused(st, Spans(False))

    def shifted():
        odd(1.0, hparams(st))
        st["t"] += 1

    ms = _interleaved([("aligned", aligned), ("odd_slot", shifted)])
    byts = kernel_bytes_per_elem("llama7b")["k_adam_step"] * S
    return {"aligned_ms": ms["aligned"], "odd_slot_ms": ms["odd_slot"],
            "odd_slot_gbs": byts / ms["odd_slot"] / 1e6,
            "odd_over_aligned_rate": ms["aligned"] / ms["odd_slot"],
            "note": "the same step with the 16-bit slot starting 2 bytes past a 4-byte word (rank r's "
                    "slot when S is odd), median of 3 alternating rounds of 5 steps"}


_CEILING = None


def ceiling_lib():
    """The benchmark's measurement kernels (libzero_ceiling.so: traffic twin, triad)."""
    global _CEILING
    if _CEILING is None:
        import ctypes
        path = os.path.join(ROOT, "zero_partition_plan_amd", "libzero_ceiling.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m zero_partition_plan_amd.build`")
        L = ctypes.CDLL(path)
        vp, u64, u32, f32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        L.zero_ceiling_twin.argtypes = [ctypes.POINTER(vp), u32, u64, vp, vp, vp, vp, f32, vp]
        L.zero_ceiling_triad.argtypes = [vp, vp, u64, f32, vp]
        L.zero_ceiling_twin.restype = L.zero_ceiling_triad.restype = ctypes.c_int
        _CEILING = L
    return _CEILING


def ceiling_context(st):
    """What this machine's memory system gives the step's own access pattern, in the same process and
    on the step's own arrays in its arena: the fused step's traffic twin (the same 11 read and 4
    write streams and bytes, trivial arithmetic) and a 2:1 in-place triad over master and m (two
    fp32 reads, one write), timed in alternation with the step. Both leave the data unchanged."""
    import ctypes

    import torch
    L = ceiling_lib()
    inp, S = st["inp"], st["S"]
    reps = inp["reps"]
    rows = list(reps.unbind(0)) if isinstance(reps, torch.Tensor) else list(reps)
    ptrs = (ctypes.c_void_p * len(rows))(*[r.data_ptr() for r in rows])
    P, M, V = (inp[k].data_ptr() for k in ("master", "m", "v"))
    out = st["slot"].data_ptr()
    stream = torch.cuda.current_stream().cuda_stream

    def twin():
        if L.zero_ceiling_twin(ptrs, len(rows), S, P, M, V, out, 0.0, stream) != 0:
            raise RuntimeError("zero_ceiling_twin refused its arguments")

    def triad():
        if L.zero_ceiling_triad(P, M, S, 0.0, stream) != 0:
            raise RuntimeError("zero_ceiling_triad refused its arguments")

    def step():
        step_fused(st, Spans(False))

    ms = _interleaved([("step", step), ("twin", twin), ("triad", triad)])
    bpe = kernel_bytes_per_elem("llama7b")["k_adam_step"]
    step_gbs, twin_gbs, triad_gbs = bpe * S / ms["step"] / 1e6, bpe * S / ms["twin"] / 1e6, 12 * S / ms["triad"] / 1e6
    return {"step_gbs": step_gbs, "twin_gbs": twin_gbs, "twin_frac": twin_gbs / HBM_PEAK_GBS,
            "triad_gbs": triad_gbs, "triad_frac": triad_gbs / HBM_PEAK_GBS,
            "step_over_twin": step_gbs / twin_gbs,
            "note": "same process, same arena: the step's traffic twin moves the step's 42 B per "
                    "element with trivial math (this box's ceiling for that mix); the triad moves "
                    "12 B per element (2 fp32 reads : 1 write); medians of 3 alternating rounds of 5 "
                    "calls"}


def setup_gather():
    import torch

    import zero_partition_plan_amd as Z
    from workloads import WORKLOADS, layer_ranges

    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    S = plan.shard_elems
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    flat = torch.randn(plan.padded_n, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    layers = layer_ranges("llama-7b")
    assert len(layers) == GATHER_LAYERS
    biggest = max(e - s for _, s, e in layers)
    log(f"workload gather7b: {len(layers)} layers, largest {biggest}, S={S}")
    st = dict(w=w, S=w.n, flat=flat, shards=[flat[r * S:(r + 1) * S] for r in range(w.nd)],
              layers=layers, bufs=[torch.empty(biggest, dtype=torch.bfloat16, device=dev) for _ in range(2)],
              t=1)
    torch.cuda.synchronize()
    return st


def step_gather(st, spans):
    """One ZeRO-3 forward's worth of gathers: every layer in order, alternating two buffers."""
    import zero_partition_plan_amd as Z
    for i, (_, a, b) in enumerate(st["layers"]):
        spans("k_gather", lambda: Z.zero_gather_params(st["shards"], a, b - a, st["bufs"][i % 2]))


def gather_prefetch_context(st, tokens: int = 1024, reps: int = 3):
    """ZeRO-3's layer pipeline on two streams: layer i computes on the current stream while layer i+1
    is gathered into the other buffer on a second stream. Events make each compute wait for its
    gather and each gather wait until the compute that last read its buffer is done (the buffer is
    released). The compute is a stand-in with no model behind it: a bf16 product of a [tokens, 4096]
    block with the layer's gathered weights viewed as [4096, k]."""
    import torch

    import zero_partition_plan_amd as Z
    layers, bufs, shards = st["layers"], st["bufs"], st["shards"]
    comp, gat = torch.cuda.current_stream(), torch.cuda.Stream()      # default priority
    x = torch.randn(tokens, 4096, device="cuda").to(torch.bfloat16)
    flops = sum(2 * tokens * (b - a) for _, a, b in layers)

    def gather(i, stream):
        _, a, b = layers[i]
        Z.zero_gather_params(shards, a, b - a, bufs[i % 2], stream=stream)

    def compute(i):
        _, a, b = layers[i]
        return torch.mm(x, bufs[i % 2][:b - a].view(4096, -1))

    def pipelined():
        ready = [torch.cuda.Event(), torch.cuda.Event()]
        free = [torch.cuda.Event(), torch.cuda.Event()]
        gat.wait_stream(comp)
        gather(0, gat)
        ready[0].record(gat)
        for i in range(len(layers)):
            if i + 1 < len(layers):
                if i >= 1:
                    gat.wait_event(free[(i + 1) % 2])   # compute i-1 has finished with that buffer
                gather(i + 1, gat)
                ready[(i + 1) % 2].record(gat)
            comp.wait_event(ready[i % 2])
            compute(i)
            free[i % 2].record(comp)
        comp.wait_stream(gat)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = new_event(True), new_event()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g_ms = timed(lambda: [gather(i, comp) for i in range(len(layers))])
    c_ms = timed(lambda: [compute(i) for i in range(len(layers))])
    p_ms = timed(pipelined)
    return {"gather_only_ms": g_ms, "compute_only_ms": c_ms, "pipelined_ms": p_ms,
            "gather_hidden": max(0.0, min(1.0, (g_ms + c_ms - p_ms) / g_ms)),
            "compute_tflops": flops / c_ms / 1e9, "tokens": tokens,
            "note": "34 layers; compute on the current stream, gathers on a second stream, two "
                    "alternating layer buffers; gather_hidden = share of the gather time the "
                    "pipeline hides. The local gather is a full-bandwidth HBM copy and contends with "
                    "the product for HBM and CUs, so on one GPU the pipeline is slower than gathering "
                    "then computing; a gather arriving over xGMI would load local HBM far less"}


def setup_offload(direct: bool = False):
    import torch

    import zero_partition_plan_amd as Z
    from workloads import WORKLOADS
    from workloads import device as D

    w = WORKLOADS["llama7b"]
    plan = Z.zero_partition_plan(w.n, w.nd)
    begin, valid = Z.zero_shard_range(plan, w.ranks[0])
    S = plan.shard_elems
    dev = torch.device("cuda:0")
    inp = D.rank_inputs(w, begin, S, valid, device=dev)
    host = {k: inp[k].cpu().numpy() for k in ("master", "m", "v")}   # the state lives on the host
    del inp["master"], inp["m"], inp["v"]
    torch.cuda.empty_cache()
    log(f"workload offload7b: S={S}, host state {3 * 4 * S / 1e9:.1f} GB, chunk {OFFLOAD_CHUNK}, "
        f"staging {'direct' if direct else 'copy'}")
    st = dict(w=w, S=S, reps=inp["reps"], host=host, t=w.warm_steps + 1,
              slot=torch.zeros(S, dtype=torch.bfloat16, device=dev), direct=direct,
              bufs=Z.offload_buffers(OFFLOAD_CHUNK, threads=OFFLOAD_THREADS, direct=direct))
    torch.cuda.synchronize()
    return st


def step_offload(st, spans):
    import zero_partition_plan_amd as Z
    h = st["host"]
    spans("offload", lambda: Z.zero_offload_step(st["reps"], st["S"], 1.0, h["master"], h["m"], h["v"],
                                                 hparams(st), st["slot"], st["bufs"]))
    st["t"] += 1


def cold_launches(st, reps=10):
    """The fused step timed after a 1 GiB scratch write that evicts the 256 MB MALL (cold caches)."""
    import torch

    import zero_partition_plan_amd as Z
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    inp, S = st["inp"], st["S"]
    ms = []
    for _ in range(reps):
        scratch.fill_(1.0)
        e0, e1 = new_event(True), new_event()
        Z.zero_adam_shard_step(inp["reps"], S, 1.0, inp["master"], inp["m"], inp["v"], hparams(st),
                               out=st["slot"])
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scratch
    return ms


def graph_steps(st, steps=50):
    """The fused step captured once in a graph with its grad scale, step counter and constants table
    on the device (zero_adam_shard_step_dev_t), replayed as successive steps, against the same
    number of eager steps through AdamStep: ms per step of each, for shards small enough that
    launch overhead shows."""
    import torch

    import zero_partition_plan_amd as Z
    w, inp, S = st["w"], st["inp"], st["S"]
    hp = Z.adam_hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                        weight_decay=w.weight_decay, wd_mode=w.wd_mode)
    table = Z.adam_table(hp, st["t"] + 2 * steps + 8)
    gs = torch.ones(1, device="cuda")
    t_dev = torch.full((1,), st["t"], dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def one():
        Z.zero_adam_shard_step_dev_t(inp["reps"], S, gs, table, t_dev, status, inp["master"], inp["m"],
                                     inp["v"], wd_mode=w.wd_mode, out=st["slot"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()                              # warm the library off the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = new_event(True), new_event()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    assert int(status.item()) == 0, "a replayed step ran past its constants table"
    st["t"] = int(t_dev.item())
    eager = Spans(False)
    step_fused(st, eager)
    torch.cuda.synchronize()
    e0, e1 = new_event(True), new_event()
    for _ in range(steps):
        step_fused(st, eager)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    del graph
    return {"graph_ms_per_step": graph_ms, "eager_ms_per_step": eager_ms, "steps": steps,
            "note": "one captured step (the update and the on-device step advance) replayed as "
                    "successive steps, against as many eager calls through the Python binding"}


def copy_ceiling(gib: int = 4):
    """A plain device copy of `gib` GiB by the library's own copy kernel (one shard, gathered whole)."""
    import torch

    import zero_partition_plan_amd as Z
    n = (gib << 30) // 2
    src = torch.empty(n, dtype=torch.int16, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    for _ in range(2):
        Z.zero_gather_params([src], 0, n, dst)
    e0, e1 = new_event(True), new_event()
    for _ in range(5):
        Z.zero_gather_params([src], 0, n, dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del src, dst
    return {"bytes_read_and_written": 2 * 2 * n, "gbs": 4 * n / ms / 1e6,
            "note": f"k_gather copying one contiguous {gib} GiB array (practical ceiling of a 1:1 copy)"}


def offload_parts(st, context: bool = True):
    """Rates of the offloaded step's parts measured alone: host update, D2H, H2D (one chunk); with
    ``context``, also the reduce kernel writing a chunk into host memory and whole steps with either
    staging, interleaved (these launch k_reduce at the host link's pace, so a profiled run skips
    them)."""
    import torch

    import zero_partition_plan_amd as Z
    C, h, b = OFFLOAD_CHUNK, st["host"], st["bufs"]
    out = torch.empty(C, dtype=torch.int16, pin_memory=True)
    t0 = time.perf_counter()
    for _ in range(3):
        Z.zero_host_adam_step(b["h_grad"], C, 1.0, h["master"][:C], h["m"][:C], h["v"][:C], hparams(st),
                              out=out, threads=OFFLOAD_THREADS)
    host_s = (time.perf_counter() - t0) / 3
    d_src = b["d_grad"] if b["d_grad"] is not None else torch.empty(C, dtype=torch.float32, device="cuda")
    e0, e1 = new_event(), new_event()
    e0.record()
    for _ in range(3):
        b["h_grad"][:C].copy_(d_src[:C], non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    d2h_ms = e0.elapsed_time(e1) / 3
    e0.record()
    for _ in range(3):
        st["slot"][:C].view(torch.int16).copy_(b["h_param"][:C], non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_ms = e0.elapsed_time(e1) / 3
    parts = {"chunk_elems": C, "host_threads": OFFLOAD_THREADS,
             "host_update_gbs": 30 * C / host_s / 1e9, "host_update_params_per_s": C / host_s,
             "d2h_gbs": 4 * C / d2h_ms / 1e6, "h2d_gbs": 2 * C / h2d_ms / 1e6,
             "note": "host update moves 30 B per element in host memory (grad 4 + state 12 read, "
                     "state 12 + bf16 2 written); d2h copies the fp32 gradient, h2d the bf16 parameters"}
    if not context:
        return parts
    # the reduce kernel writing one chunk straight into pinned host memory
    chunk = [r[:C] for r in st["reps"]]
    h_g = b["h_grad"][:C]
    Z.zero_reduce_shard(chunk, C, h_g)
    e0.record()
    for _ in range(3):
        Z.zero_reduce_shard(chunk, C, h_g)
    e1.record()
    torch.cuda.synchronize()
    kd2h_ms = e0.elapsed_time(e1) / 3
    # whole steps with either staging, interleaved, on the same state
    other = Z.offload_buffers(C, threads=OFFLOAD_THREADS, direct=not st["direct"])
    both = {("direct" if st["direct"] else "copy"): b, ("copy" if st["direct"] else "direct"): other}
    times = {k: [] for k in both}
    for _ in range(4):
        for k, bb in both.items():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            Z.zero_offload_step(st["reps"], st["S"], 1.0, h["master"], h["m"], h["v"], hparams(st),
                                st["slot"], bb)
            times[k].append((time.perf_counter() - t0) * 1e3)
            st["t"] += 1
    del other
    parts["d2h_by_kernel_gbs"] = 4 * C / kd2h_ms / 1e6
    parts["step_ms_by_staging"] = {k: round(sorted(v)[len(v) // 2], 2) for k, v in times.items()}
    parts["note"] += ("; d2h_by_kernel: the reduce kernel writes the chunk into pinned host memory "
                      "itself; step_ms_by_staging: the upper median of 4 whole steps each, interleaved")
    return parts


def hparams(st):
    import zero_partition_plan_amd as Z
    w = st["w"]
    return Z.adam_hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                          weight_decay=w.weight_decay, wd_mode=w.wd_mode, step=st["t"])


class Spans:
    """HIP-event pairs around library calls, per kernel name, on the stream the library uses.

    The events are created before the timed region (``reserve`` pairs, more in blocks if needed),
    so that a span costs the host two event records and nothing else: with launches of ~0.1 ms the
    host must stay ahead of the GPU, or the GPU idles inside a span and the span overstates the
    kernel's time.
    """

    def __init__(self, on: bool, reserve: int = 0):
        self.on = on
        self.pairs = {}
        self.pool = [(new_event(), new_event()) for _ in range(reserve)] if on else []
        self.used = 0

    def __call__(self, name, fn):
        if not self.on:
            return fn()
        if self.used == len(self.pool):
            self.pool += [(new_event(), new_event()) for _ in range(256)]
        a, b = self.pool[self.used]
        self.used += 1
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]

    def relabel_last(self, name, new_name):
        """File the last span of ``name`` under ``new_name`` instead."""
        if self.on and self.pairs.get(name):
            self.pairs.setdefault(new_name, []).append(self.pairs[name].pop())


def step_fused(st, spans):
    """One step of a fused workload: one launch per window (one window unless the shard is windowed)."""
    import zero_partition_plan_amd as Z
    inp, S, W = st["inp"], st["S"], st["w"].window
    if "calls" not in st:              # arrays marshalled once: a step passes only its scalars
        st["calls"] = [Z.AdamStep(inp["reps"], min(S, a + (W or S)) - a, inp["master"][a:],
                                  inp["m"][a:], inp["v"][a:], out=st["slot"][a:])
                       for a in range(0, S, W or S)]
    h = hparams(st)
    for call in st["calls"]:
        spans("k_adam_step", lambda: call(1.0, h))
    st["t"] += 1


def step_two_pass(st, spans):
    """Reduce -> squared norm -> clip scale -> AdamW, all enqueued on the device with nothing read
    back between the passes: zero_clip_scale forms the grad scale from the device norm, and the
    update reads it and the overflow flag from device memory (a flagged step writes nothing).

    The host learns a step's flag one step late, from a 4-byte copy enqueued after its reduce pass:
    the next step waits for that copy (the GPU meanwhile runs this step's update), and t advances
    only past steps that were not skipped.
    """
    import zero_partition_plan_amd as Z
    resolve_two_pass(st)
    w, inp, S = st["w"], st["inp"], st["S"]
    inv_ls = 1.0 / w.loss_scale
    st["flag"].zero_()
    spans("k_reduce", lambda: Z.zero_reduce_shard(inp["reps"], S, st["g"], st["flag"], st["parts"],
                                                  inv_ls))
    st["host_flag"].copy_(st["flag"], non_blocking=True)
    st["flag_ready"].record()
    Z.zero_shard_sqnorm(None, S, inv_ls, st["parts"], st["sq"])
    Z.zero_clip_scale(st["sq"], w.max_norm, 1e-6, inv_ls, st["gs"])
    spans("k_adam_step", lambda: Z.zero_adam_shard_step_dev_scale(
        [st["g"]], S, st["gs"], inp["master"], inp["m"], inp["v"], hparams(st), out=st["slot"],
        skip=st["flag"]))
    st["flag_pending"] = spans


def resolve_two_pass(st):
    """Account for the last two-pass step once its flag is on the host: t advances unless it was
    skipped; a skipped step's update launch (which exits at once) is timed apart from real ones."""
    spans = st.get("flag_pending")
    if spans is None:
        return
    st["flag_ready"].synchronize()
    st["flag_pending"] = None
    if int(st["host_flag"][0]):
        st["skipped"] += 1
        spans.relabel_last("k_adam_step", "k_adam_step_skipped")
    else:
        st["t"] += 1


def new_event(record=False):
    import torch
    e = torch.cuda.Event(enable_timing=True)
    if record:
        e.record()
    return e


def pct(xs, q):
    s = sorted(xs)
    return s[min(len(s) - 1, int(round(q * (len(s) - 1))))]


# ----------------------------------------------------------------------------- CPU baseline

def _oracle_passes(name: str, seconds: float, seed_offset: int = 0):
    """Run the oracle's step over one host-drawn window of the workload until `seconds` have gone."""
    import oracle as O
    from workloads import WORKLOADS
    from workloads import host as H

    w = WORKLOADS["llama13b" if name.startswith("llama13b") else name]
    win = CPU_WINDOW
    plan = O.partition_plan(w.n, w.nd)
    begin, _ = O.shard_range(plan, w.ranks[0])
    hp = O.AdamHParams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, wd_mode=w.wd_mode, step=w.warm_steps + 1)
    inp = H.rank_inputs(w, begin, win, win, seed_offset=seed_offset)
    elems, t_used = 0, 0.0
    while t_used < seconds:
        t0 = time.perf_counter()
        O.sharded_step(list(inp["reps"]), w.rep_dtype, 1.0, inp["master"], inp["m"], inp["v"], hp,
                       w.out_dtypes[0])
        t_used += time.perf_counter() - t0
        elems += win
    return elems, t_used


def _oracle_worker(args):
    return _oracle_passes(*args)


CPU_WINDOW = 1 << 21
CPU_WORKERS = 16            # host cores: a 16-core host share per GPU


def cpu_baseline(name: str, seconds: float):
    """The oracle, as it stands, on windows of the same workload drawn on the host: one process
    (numpy ufuncs are single-threaded, so one core), then CPU_WORKERS processes side by side."""
    import multiprocessing as mp

    elems, t_used = _oracle_passes(name, seconds)
    single = elems / t_used
    workers = min(CPU_WORKERS, os.cpu_count() or 1)
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(name, seconds * 2 / 3, k + 1) for k in range(workers)])
    multi = sum(e / t for e, t in res)
    return {"value": single, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{elems // CPU_WINDOW} passes of the numpy oracle (replica sum + AdamW + cast) "
                      f"over a {CPU_WINDOW}-element window of the {name} shard drawn on the host, "
                      f"{t_used:.1f} s of one host core; host has {os.cpu_count()} logical CPUs",
            "all_cores": {"value": multi, "unit": "params/s", "cores": workers,
                          "sample": f"{workers} processes, each the same oracle on its own "
                                    f"{CPU_WINDOW}-element window for {seconds * 2 / 3:.0f} s; "
                                    f"value = sum of their rates"}}


# ----------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description="sharded ZeRO AdamW step benchmark")
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (only 1: one rank's shard on one GPU)")
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about 5 s of timed work for the workload, so that a "
                         "GPU-utilisation sampler sees the run: " +
                         ", ".join(f"{k} {v}" for k, v in DEFAULT_STEPS.items()) + ")")
    ap.add_argument("--warmup", type=int, default=3, help="untimed steps first")
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "gpt2", "llama13b", "llama13b-clean", "gpt3", "gather7b",
                             "offload7b"])
    ap.add_argument("--config", type=int, choices=[2, 3, 4, 5],
                    help="the workload by its config number: 2 gpt2, 3 llama7b, 4 llama13b, 5 gpt3 "
                         "(config 1, the tiny all-ranks case, is a correctness case for the tests)")
    ap.add_argument("--placement", default="arena", choices=["arena", "separate"],
                    help="arrays of the step in one arena laid out by zero_arena_layout, or each in "
                         "its own allocation")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context legs (copy ceiling, separate-placement step, cold launches, graph "
                         "replay, the offloaded step's direct-staging legs), "
                         "so that a profiler sees only the timed step's launches")
    ap.add_argument("--offload-staging", default="copy", choices=["copy", "direct"],
                    help="offload7b: gradient chunks reduced into device staging and copied to pinned "
                         "host memory, or written there by the reduce kernel itself")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle's CPU baseline (0 skips it)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", action="store_true",
                    help="(no GPU) write the profile summaries under profiles/ from the profile runs")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the profiling commands for --workload and exit")
    args = ap.parse_args(argv)
    if args.config is not None:
        args.workload = {2: "gpt2", 3: "llama7b", 4: "llama13b", 5: "gpt3"}[args.config]
    if args.steps is None:
        args.steps = DEFAULT_STEPS[args.workload]
    if args.profile_commands:
        for k, c in profile_commands(args.workload).items():
            print(f"{c} > {profile_dirs(args.workload)[k]}.log 2>&1")
        return 0
    if args.summarize:
        summarize(args.workload)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark measures one rank's shard "
              f"on one GPU (--gpus 1); a multi-GPU run would add the reduce-scatter and all-gather "
              f"around this step", file=sys.stderr, flush=True)
        return 2

    import torch
    import zero_partition_plan_amd as Z
    Z.lib()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    log(f"kernel source sha256[:16] {kernel_hash(dominant_kernels(args.workload)[0])}")

    if args.workload == "gather7b":
        st, step = setup_gather(), step_gather
    elif args.workload == "offload7b":
        st, step = setup_offload(args.offload_staging == "direct"), step_offload
    else:
        st = setup(args.workload, args.placement)
        step = step_two_pass if args.workload.startswith("llama13b") else step_fused
    w, S = st["w"], st["S"]

    nvtx = torch.cuda.nvtx             # roctx ranges: phases show up in a marker trace
    nvtx.range_push(f"warmup {args.workload}")
    for _ in range(args.warmup):
        step(st, Spans(False))
    torch.cuda.synchronize()
    nvtx.range_pop()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    spans = Spans(True, reserve=args.steps * launches_per_step(args.workload))
    t_start, t_end = new_event(), new_event()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()                       # no collector pause while the host enqueues the timed steps
    nvtx.range_push(f"timed {args.steps} steps {args.workload}")
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step(st, spans)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if "flag_pending" in st:
        resolve_two_pass(st)           # the last step's overflow flag
    nvtx.range_pop()
    gc.enable()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    params_per_s = S * args.steps / (total_ms / 1e3)

    kernels = dominant_kernels(args.workload)
    bpe = kernel_bytes_per_elem(args.workload)
    n_launch = launch_elems(args.workload)
    per_kernel = {}
    parts = None
    if args.workload == "offload7b":
        # the reduce kernel runs inside the offloaded call; time it alone over the chunks one step
        # walks (so the mean launch is launch_elems' and a profiled run sees only whole sequences)
        import zero_partition_plan_amd as Z
        d_g = st["bufs"]["d_grad"]
        if d_g is None:                    # direct staging: time the kernel into device memory here
            d_g = torch.empty(OFFLOAD_CHUNK, dtype=torch.float32, device="cuda")
        # (marshalled once, so that the host keeps ahead of 0.1 ms launches)
        calls = [Z.ReduceCall([r[a:min(S, a + OFFLOAD_CHUNK)] for r in st["reps"]],
                              min(S, a + OFFLOAD_CHUNK) - a, d_g) for a in range(0, S, OFFLOAD_CHUNK)]
        for call in calls:
            call()
        for _ in range(2):
            for call in calls:
                spans("k_reduce", call)
        torch.cuda.synchronize()
        parts = offload_parts(st, context=not args.no_context)
    for k in kernels:
        xs = spans.ms(k)
        if not xs:                         # e.g. the update pass of steps that were all skipped
            per_kernel[k] = {"launches": 0}
            log(f"{k}: not launched")
            continue
        per_kernel[k] = {"launches": len(xs), "avg_ms": sum(xs) / len(xs), "median_ms": pct(xs, 0.5),
                         "min_ms": min(xs), "p90_ms": pct(xs, 0.9),
                         "bytes_per_elem": bpe[k],
                         "gbs_at_avg": bpe[k] * n_launch / (sum(xs) / len(xs)) / 1e6}
        log(f"{k}: {len(xs)} launches, avg {per_kernel[k]['avg_ms']:.4f} ms, median "
            f"{per_kernel[k]['median_ms']:.4f}, min {per_kernel[k]['min_ms']:.4f}, p90 "
            f"{per_kernel[k]['p90_ms']:.4f} -> {per_kernel[k]['gbs_at_avg']:.0f} GB/s")
        if len(xs) >= 200:             # drift over a long timed region (clocks, temperature)
            q = len(xs) // 10
            log(f"{k}: first {q} launches avg {sum(xs[:q]) / q:.4f} ms, last {q} avg "
                f"{sum(xs[-q:]) / q:.4f} ms")
    if "skipped" in st:
        log(f"overflow-skipped steps: {st['skipped']} of {args.warmup + args.steps}")
        xs = spans.ms("k_adam_step_skipped")
        if xs:
            log(f"k_adam_step on a set skip flag (exits at once): {len(xs)} launches, avg "
                f"{sum(xs) / len(xs):.4f} ms")
    log(f"{args.steps} steps: {total_ms:.3f} ms on events, {wall * 1e3:.3f} ms wall")
    if "inp" in st:
        assert torch.isfinite(st["inp"]["master"][:1 << 20]).all()

    dom = kernels[0]
    achieved = per_kernel[dom]["gbs_at_avg"]
    traffic = recorded_traffic(args.workload, dom)

    cold = None
    if args.workload == "gpt2" and not args.no_context:
        cms = cold_launches(st)
        cold = {"median_ms": pct(cms, 0.5), "min_ms": min(cms), "p90_ms": pct(cms, 0.9),
                "gbs_at_median": bpe[dom] * n_launch / pct(cms, 0.5) / 1e6,
                "note": "each launch after a 1 GiB scratch write (the 256 MB MALL evicted); the "
                        "roofline figures above are warm (back-to-back launches)"}
        log(f"cold launches: median {cold['median_ms']:.4f} ms -> {cold['gbs_at_median']:.0f} GB/s")
    context = None
    if args.workload == "gpt2" and not args.no_context:
        context = {"graph": graph_steps(st)}
        gr = context["graph"]
        log(f"graph replay: {gr['graph_ms_per_step']:.4f} ms per step, eager "
            f"{gr['eager_ms_per_step']:.4f} ms per step")
    if args.workload == "gather7b" and not args.no_context:
        nvtx.range_push("context legs")
        context = {"prefetch": gather_prefetch_context(st)}
        pf = context["prefetch"]
        log(f"prefetch pipeline: gathers {pf['gather_only_ms']:.3f} ms, compute {pf['compute_only_ms']:.3f} "
            f"ms, pipelined {pf['pipelined_ms']:.3f} ms; {100 * pf['gather_hidden']:.0f}% of the gather "
            f"time hidden")
        nvtx.range_pop()
    if args.workload == "llama7b" and not args.no_context:
        nvtx.range_push("context legs")
        context = {"copy_ceiling": copy_ceiling()}
        log(f"copy ceiling: {context['copy_ceiling']['gbs']:.0f} GB/s")
        context["odd_slot"] = odd_slot_context(st)
        log(f"odd slot: {context['odd_slot']['odd_slot_ms']:.4f} ms per step against "
            f"{context['odd_slot']['aligned_ms']:.4f} aligned")
        if args.placement == "arena":
            context["ceiling"] = ceiling_context(st)
            c = context["ceiling"]
            log(f"same-arena ceilings: step {c['step_gbs']:.0f} GB/s, traffic twin {c['twin_gbs']:.0f} "
                f"GB/s ({100 * c['twin_frac']:.1f}% of peak), triad {c['triad_gbs']:.0f} GB/s; "
                f"step / twin {c['step_over_twin']:.3f}")
            context["placement"] = placement_context(args.workload)
            log(f"separate allocations: {context['placement']['separate_ms_per_step']:.4f} ms per step")
        nvtx.range_pop()

    if args.copy_calib:
        nb = args.copy_calib << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 x {nb} bytes read + {nb} bytes written")
        del src, dst

    cpu = None
    if args.cpu_seconds > 0 and args.workload not in ("gather7b", "offload7b"):
        log(f"cpu baseline: oracle for {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    line = {
        "metric": {"gather7b": "ZeRO-3 layer gather params/s + achieved HBM GB/s vs peak (7B, Nd=8)",
                   "offload7b": "ZeRO-Offload sharded Adam step params/s (7B, Nd=8, host-resident state)"
                   }.get(args.workload, METRIC),
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.workload != "gather7b" else "bf16",
        "data": "synthetic (seeded device draws; model shapes only, no weights)",
        "config": ({
            "workload": WL_DESC[args.workload],
            "params_gathered_per_step": S,
            "shards": w.nd,
            "layers": GATHER_LAYERS,
            "dtype": "bf16",
            "launches_per_step": {k: v["launches"] // args.steps for k, v in per_kernel.items()},
        } if args.workload == "gather7b" else {
            "workload": WL_DESC[args.workload],
            "shard_elems": S,
            "replicas": w.reps,
            "replica_dtype": w.rep_dtype,
            "param_out_dtype": w.out_dtypes[0],
            "optimizer": f"AdamW wd={w.weight_decay}",
            "placement": st.get("placement"),
            "first_timed_t": w.warm_steps + 1 + args.warmup,
            "launches_per_step": ({"k_reduce": -(-S // OFFLOAD_CHUNK)} if args.workload == "offload7b"
                                  else {k: v["launches"] / args.steps for k, v in per_kernel.items()}),
            **({"overflow_skipped_steps": st["skipped"], "counted_steps": args.warmup + args.steps}
               if "skipped" in st else {}),
        }),
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bpe[dom] * n_launch,
            "avg_launch_ms": per_kernel[dom]["avg_ms"],
            "launch_ms": {k: {q: round(v[q], 5) for q in ("median_ms", "min_ms", "p90_ms")}
                          for k, v in per_kernel.items() if v["launches"]},
        },
        "cpu_baseline": cpu,
    }
    if parts is not None:
        line["offload"] = parts
    if cold is not None:
        line["cold"] = cold
    if context is not None:
        line["context"] = context
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
