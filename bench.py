#!/usr/bin/env python3
"""Throughput of one data-parallel rank's sharded AdamW step on one MI355X.

Default workload: the Llama-7B-shaped flat parameter space (6,738,415,616 elements) over Nd = 8
ranks, one rank's 842,301,952-element shard: 8 bf16 gradient replicas summed in fixed order,
AdamW on the fp32 master / m / v (warm state, t = 11), bf16 cast into the rank's slot of the full
gathered parameter buffer. One step = one fused kernel launch. Inputs are drawn on the device and
are resident in HBM before the timed region.

Prints one JSON line (see the fields below). Flags:
  --gpus N         only 1 is supported: this path runs on one GPU's shard
  --steps K        timed steps (default 20)
  --warmup W       untimed steps first (default 3)
  --workload NAME  llama7b (default), gpt2, llama13b (two-pass clip path), gpt3 (64 Mi windows)
  --cpu-seconds S  budget of the oracle's CPU baseline (default 12; 0 skips it)
  --copy-calib MB  also run a plain device copy of MB MiB 5 times (for counter calibration)
"""

from __future__ import annotations

import argparse
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
KERNEL_SRC = os.path.join(ROOT, "zero_partition_plan_amd", "csrc", "zero_step.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


# ----------------------------------------------------------------------------- workloads

def setup(name: str):
    import torch

    import zero_partition_plan_amd as Z
    from workloads import WORKLOADS
    from workloads import device as D

    w = WORKLOADS[name]
    plan = Z.zero_partition_plan(w.n, w.nd)
    rank = w.ranks[0]
    begin, valid = Z.zero_shard_range(plan, rank)
    S = plan.shard_elems
    dev = torch.device("cuda:0")
    log(f"workload {name}: N={w.n} Nd={w.nd} rank={rank} S={S} R={w.reps}x{w.rep_dtype}")
    inp = D.rank_inputs(w, begin, S, valid, device=dev, rep_size=w.window)
    out_t = torch.float16 if w.out_dtypes[0] == "f16" else torch.bfloat16
    state = dict(w=w, plan=plan, S=S, begin=begin, inp=inp, t=w.warm_steps + 1)
    if w.window is None and name != "llama13b":
        state["full"] = torch.zeros(plan.padded_n, dtype=out_t, device=dev)
        state["slot"] = state["full"][begin:begin + S]
    else:
        state["slot"] = torch.zeros(S, dtype=out_t, device=dev)
    if name == "llama13b":
        state["g"] = torch.empty(S, device=dev)
        state["flag"] = torch.zeros(1, dtype=torch.int32, device=dev)
        state["parts"] = torch.empty(Z.ZERO_SQ_PARTIALS, dtype=torch.float64, device=dev)
        state["sq"] = torch.empty(1, dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    return state


def hparams(st):
    import zero_partition_plan_amd as Z
    w = st["w"]
    return Z.adam_hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                          weight_decay=w.weight_decay, wd_mode=w.wd_mode, step=st["t"])


def step_fused(st, events=None):
    """One step of a fused workload; returns the number of kernel launches."""
    import zero_partition_plan_amd as Z
    inp, S, W = st["inp"], st["S"], st["w"].window
    h = hparams(st)
    launches = 0
    for a in range(0, S, W or S):
        b = min(S, a + (W or S))
        if events is not None:
            events.append(new_event(True))
        Z.zero_adam_shard_step(inp["reps"], b - a, 1.0, inp["master"][a:], inp["m"][a:], inp["v"][a:],
                               h, out=st["slot"][a:])
        if events is not None:
            events.append(new_event(True))
        launches += 1
    st["t"] += 1
    return launches


def step_two_pass(st, events=None):
    """Reduce -> squared norm -> clip scale (host) -> AdamW with the device skip flag."""
    import zero_partition_plan_amd as Z
    w, inp, S = st["w"], st["inp"], st["S"]
    inv_ls = 1.0 / w.loss_scale
    st["flag"].zero_()
    Z.zero_reduce_shard(inp["reps"], S, st["g"], st["flag"], st["parts"], inv_ls)
    Z.zero_shard_sqnorm(None, S, inv_ls, st["parts"], st["sq"])
    sq = float(st["sq"].item())                 # 8-byte device -> host read for the clip scale
    coef = min(1.0, w.max_norm / (math.sqrt(sq) + 1e-6)) if math.isfinite(sq) else 1.0
    if events is not None:
        events.append(new_event(True))
    Z.zero_adam_shard_step([st["g"]], S, coef * inv_ls, inp["master"], inp["m"], inp["v"],
                           hparams(st), out=st["slot"], skip=st["flag"])
    if events is not None:
        events.append(new_event(True))
    st["t"] += 1
    return 1


def new_event(record=False):
    import torch
    e = torch.cuda.Event(enable_timing=True)
    if record:
        e.record()
    return e


def bytes_per_param(w, two_pass=False):
    rb = {"f32": 4, "f16": 2, "bf16": 2}[w.rep_dtype]
    if two_pass:
        return 4 + 24 + 2            # the Adam launch alone reads the fp32 gradient
    return w.reps * rb + 24 + 2


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(name: str, seconds: float):
    """The oracle, as it stands, on windows of the same workload drawn on the host."""
    import numpy as np

    import oracle as O
    from workloads import WORKLOADS
    from workloads import host as H

    w = WORKLOADS[name]
    win = 1 << 21
    plan = O.partition_plan(w.n, w.nd)
    begin, _ = O.shard_range(plan, w.ranks[0])
    hp = O.AdamHParams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, wd_mode=w.wd_mode, step=w.warm_steps + 1)
    inp = H.rank_inputs(w, begin, win, win)
    elems, t_used = 0, 0.0
    while t_used < seconds:
        t0 = time.perf_counter()
        O.sharded_step(list(inp["reps"]), w.rep_dtype, 1.0, inp["master"], inp["m"], inp["v"], hp,
                       w.out_dtypes[0])
        t_used += time.perf_counter() - t0
        elems += win
    return {"value": elems / t_used, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{elems // win} passes of the numpy oracle (replica sum + AdamW + cast) over a "
                      f"{win}-element window of the {name} shard drawn on the host, "
                      f"{t_used:.1f} s of one host core (numpy ufuncs are single-threaded); "
                      f"host has {os.cpu_count()} logical CPUs"}


# ----------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description="sharded ZeRO AdamW step benchmark")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b", choices=["llama7b", "gpt2", "llama13b", "gpt3"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calib", type=int, default=0)
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build measures one rank's shard "
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

    st = setup(args.workload)
    two_pass = args.workload == "llama13b"
    step = step_two_pass if two_pass else step_fused
    w, S = st["w"], st["S"]

    for _ in range(args.warmup):
        step(st)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    kernel_events = []
    t_start = new_event()
    t_end = new_event()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    launches = 0
    for _ in range(args.steps):
        launches += step(st, kernel_events)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    k_ms = [kernel_events[i].elapsed_time(kernel_events[i + 1]) for i in range(0, len(kernel_events), 2)]
    avg_launch_ms = sum(k_ms) / len(k_ms)
    ms_per_step = total_ms / args.steps
    params_per_s = S * args.steps / (total_ms / 1e3)
    log(f"{args.steps} steps: {total_ms:.3f} ms on events, {wall * 1e3:.3f} ms wall; "
        f"adam launch avg {avg_launch_ms:.4f} ms (min {min(k_ms):.4f}, max {max(k_ms):.4f})")
    assert torch.isfinite(st["inp"]["master"][:1 << 20]).all()

    bpp = bytes_per_param(w, two_pass)
    elems_per_launch = S * args.steps / launches
    achieved = bpp * elems_per_launch / (avg_launch_ms / 1e3) / 1e9
    kernel_name = "k_adam_step"
    traffic = recorded_traffic(args.workload, kernel_name)

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
    if args.cpu_seconds > 0:
        log(f"cpu baseline: oracle for {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    wl_desc = {
        "llama7b": "Llama-7B-shaped flat space (6,738,415,616 params), Nd=8, rank 0 shard",
        "gpt2": "GPT-2-small-shaped flat space (124,356,864 params), Nd=8, rank 3 shard",
        "llama13b": "Llama-13B-shaped flat space (13,015,864,320 params), Nd=16, rank 5 shard, two-pass clip path",
        "gpt3": "GPT-3-175B-shaped flat space (174,604,259,328 params), Nd=64, rank 0 shard in 64 Mi windows",
    }[args.workload]
    line = {
        "metric": METRIC,
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded device draws; model shapes only, no weights)",
        "config": {
            "workload": wl_desc,
            "shard_elems": S,
            "replicas": w.reps,
            "replica_dtype": w.rep_dtype,
            "param_out_dtype": w.out_dtypes[0],
            "optimizer": f"AdamW wd={w.weight_decay}",
            "first_timed_t": w.warm_steps + 1 + args.warmup,
            "launches_per_step": launches // args.steps,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_param": bpp,
            "avg_launch_ms": avg_launch_ms,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
