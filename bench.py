#!/usr/bin/env python3
"""Throughput of the SDM recurrent core (select + gated delta write + sparse
read) on one MI355X, on the seeded synthetic workload.

    python bench.py [--steps K] [--warmup W] [--workload 1] [--gpus 1]

A step is one sdm_forward over the whole workload (M <- M_0, selection of
every head-token, then the write/read recurrence over all tokens); value is
head-tokens per second over K such steps.  A second pass of K steps issues
each step as sdm_prepare + sdm_apply on one stream, so that HIP events on the
launch stream time the write/read phase on its own (roofline).  Inputs are
resident in HBM before timing.  Prints one JSON line.

roofline: HBM-bound; achieved = algorithmic row bytes of the step (per
head-token (W + R) row reads + W row writes of d_v float32) / the write/read
phase's duration; traffic = the same phase's HBM bytes from rocprofv3
FETCH_SIZE / WRITE_SIZE counters, scaled by a copy kernel of known size
(profiles/), or null when the kernel source changed since.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
FP8_SCALE_LOG2 = -4  # E4M3 state: codes of M * 2^4 (magnitudes up to 28)
METRIC = "SDM select+write+read head-tokens/s and achieved HBM GB/s (% peak)"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


SCHEDULES = {  # schedule -> (kernel source, kernels of the write/read phase)
    "token-serial": ("rw_serial.hip", "rw_serial_kernel, or rw_split_kernel where the (chain, "
                                      "slice) units are fewer than four per compute unit (one launch)"),
    "time-parallel": ("rw_timepar.hip", "tp_read_kernel + tp_update_kernel (one pair per epoch)"),
}
# a bfloat16 or E4M3 state: the library's choice for the shape
NARROW_KERNELS = ("tp_fused_stored_kernel (one launch: every epoch's reads, then its writes) "
                  "where the epochs fit its LDS and the (chain, slice) units fill the GPU, else "
                  "tp_read_stored_kernel + tp_update_kernel (one pair per epoch)")


def rw_kernels(schedule, state):
    """What runs the write/read phase, for the roofline's `kernel` field."""
    if schedule == "time-parallel" and state != "f32":
        return NARROW_KERNELS
    return SCHEDULES[schedule][1]


# headers every kernel source includes: a change there changes the kernels too
KERNEL_HEADERS = ("sdm_internal.h", "tp_device.h")


def kernel_source_hash(schedule, root=None):
    """sha256 over the schedule's kernel source and the headers it includes
    (a missing file counts as changed content)."""
    csrc = os.path.join(root or ROOT, "sparse_memory_linear_select_amd", "csrc")
    h = hashlib.sha256()
    for name in (SCHEDULES[schedule][0],) + KERNEL_HEADERS:
        h.update(name.encode() + b"\0")
        try:
            h.update(open(os.path.join(csrc, name), "rb").read())
        except OSError:
            h.update(b"<missing>")
    return h.hexdigest()


def _traffic(wl, schedule, state="f32"):
    """Counter-measured HBM bytes of the write/read phase per step, if a
    committed summary exists for this workload, schedule and state type and
    the kernel source is unchanged since the counters were taken; else None."""
    tag = schedule.replace("-", "_") + "__" + wl.name.replace(" ", "_")
    if state != "f32":
        tag += f"__{state}_state"
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != kernel_source_hash(schedule):
            return None
        return float(rec["hbm_bytes_per_step"])
    except Exception:
        return None


def d2d_copy_gbs(dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate (read + write bytes / time) of a 1 GiB
    buffer: the practical streaming ceiling of this GPU's HBM."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (virtual machines often give only a short name)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                    info[k] = v
            elif info:
                break  # end of the first processor's block
    except OSError:
        pass
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(d, wl, seqs, T=None, state="f32", threads=None, runs=5):
    """The float64 oracle on a bounded sample of the same inputs (the first
    `seqs` sequences, their first T tokens): select + init + recurrence,
    median wall time of `runs` runs on `threads` host threads (all by
    default)."""
    import statistics

    import numpy as np

    import oracle

    T = wl.T if T is None else min(T, wl.T)
    sub = {k: (np.ascontiguousarray(v[:seqs, :T]) if k != "M0" else v) for k, v in d.items()
           if k != "src"}
    cores = threads or oracle.default_threads()
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle.forward(sub, wl.sqrtN, wl.W, wl.R, threads=cores, state=state,
                       scale_log2=FP8_SCALE_LOG2)
        times.append(time.perf_counter() - t)
    dt = statistics.median(times)
    ht = seqs * T * wl.H
    return {"value": ht / dt, "unit": "head-tokens/s", "cores": cores, "kind": "oracle",
            "cpu": _cpu_model(), "runs": runs,
            "sample": f"{wl.name}: {seqs} of {wl.B} sequences x {T} of {wl.T} tokens x {wl.H} "
                      f"heads ({ht} head-tokens, all {wl.d_v} columns), select + init + "
                      f"recurrence, median of {runs} runs: {dt:.3f} s"}


def measure_decode(wl, steps, warm, variant="auto"):
    """B sequences advance by one token per call (T = 1), continuing from the
    state left by a 256-token prefill: the step latency issued eagerly and
    replayed from a captured HIP graph."""
    import numpy as np
    import torch

    import sdm_inputs as si
    import sparse_memory_linear_select_amd as sdm

    prefix = 256
    d = si.generate(wl, T=prefix + warm + steps)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    core = sdm.SDM(up(d["M0"]), wl.W, wl.R)
    names = ("kp", "qp", "v", "alpha", "beta")
    pre = [up(d[n][:, :prefix]) for n in names]
    var = {"auto": sdm.AUTO, "serial": sdm.SERIAL, "timepar": sdm.TIMEPAR}[variant]
    _, M = core.forward(*pre, variant=var)
    toks = [[up(d[n][:, t:t + 1]) for n in names] for t in range(prefix, prefix + warm + steps)]
    dt_code = sdm.BF16 if wl.dtype == "bf16" else sdm.F32
    ws = torch.empty(core.workspace_size(wl.B, 1, dt_code, var), dtype=torch.uint8, device=dev)
    y = torch.empty((wl.B, 1, wl.H, wl.d_v), dtype=torch.float32, device=dev)
    for t in range(warm):
        core.forward(*toks[t], variant=var, y=y, M=M, workspace=ws, cont=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warm, warm + steps):
        core.forward(*toks[t], variant=var, y=y, M=M, workspace=ws, cont=True)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the same steps captured once in a HIP graph and replayed (no per-launch
    # host overhead): what a serving loop that replays captured steps pays
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(warm, warm + steps):
            core.forward(*toks[t], variant=var, y=y, M=M, workspace=ws, cont=True)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / steps
    schedule = sdm.variant_name(core, wl.B, 1, dt_code, var)
    del g, toks, pre, M, ws, y, core
    torch.cuda.empty_cache()
    return {"us_per_step": us, "graph_replay_us_per_step": us_graph, "steps": steps,
            "warmup": warm, "prefill_tokens": prefix, "schedule": schedule}


def decode(args, wl):
    """Decode: B sequences advance by one token per call (T = 1), continuing
    from the state left by a 256-token prefill.  Reports the step latency."""
    r = measure_decode(wl, args.steps * 20, args.warmup * 5, args.variant)
    print(json.dumps({
        "metric": "SDM decode step latency (one token for each of B sequences, state continued)",
        "value": r["us_per_step"], "unit": "us/step", "higher_is_better": False, "n_gpus": 1,
        "steps": r["steps"], "warmup": r["warmup"],
        "head_tokens_per_s": wl.B * wl.H / (r["us_per_step"] * 1e-6),
        "graph_replay_us_per_step": r["graph_replay_us_per_step"],
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "sqrtN": wl.sqrtN, "d_v": wl.d_v,
                   "W": wl.W, "R": wl.R, "prefill_tokens": r["prefill_tokens"],
                   "schedule": r["schedule"]},
        "data": "synthetic (seeded; recipe in sdm_inputs.py)"}), flush=True)


def backward(args, wl):
    """Backward of the core over the whole workload: dL/dy random, dL/dM_T
    random; one step = one sdm_backward call (it recomputes the forward)."""
    import numpy as np
    import torch

    import sdm_inputs as si
    import sparse_memory_linear_select_amd as sdm

    d = si.generate(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    dd = {k: up(v) for k, v in d.items() if k != "src"}
    core = sdm.SDM(dd["M0"], wl.W, wl.R)
    args_ = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    g = torch.Generator(device=dev).manual_seed(0)
    dy = torch.randn((wl.B, wl.T, wl.H, wl.d_v), device=dev, generator=g)
    dMT = torch.randn((wl.B, wl.H, wl.N, wl.d_v), device=dev, generator=g)
    dt_code = sdm.BF16 if wl.dtype == "bf16" else sdm.F32
    nb = core.backward_workspace_size(wl.B, wl.T, dt_code, args.backward_chunks)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        core.backward(*args_, dy, dMT=dMT, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        core.backward(*args_, dy, dMT=dMT, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({
        "metric": "SDM backward head-tokens/s (forward recompute + reverse, selections fixed)",
        "value": wl.head_tokens / (ms * 1e-3), "unit": "head-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "workspace_gb": nb / 1e9,
        "chunks": args.backward_chunks or "least memory",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "sqrtN": wl.sqrtN,
                   "d_v": wl.d_v, "W": wl.W, "R": wl.R, "inputs": wl.dtype},
        "data": "synthetic (seeded; recipe in sdm_inputs.py)"}), flush=True)


def _short_kernel(name: str) -> str:
    """`tp_read_kernel<16, false>` from a demangled rocprofv3 kernel name."""
    import re

    name = re.sub(r"^void ", "", name.strip())
    name = re.sub(r"\(anonymous namespace\)::|sdm::", "", name)
    depth, out = 0, []
    for ch in name:  # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    short = "".join(out).strip()
    if len(short) > 100:  # a library kernel's long template arguments
        short = short[:short.index("<")] + "<...>" if "<" in short else short[:100] + "..."
    return short


def counters_summary(args, wl):
    """Summarise rocprofv3 `--pmc` runs of this script (CSV output, one
    directory per run): per kernel, the number of dispatches and the mean of
    every counter per dispatch, as a markdown table on stdout.  When the runs
    hold FETCH_SIZE and WRITE_SIZE, also write the workload's counted HBM
    traffic of the write/read phase (profiles/traffic_*.json, the `traffic`
    of the JSON line): both counters are scaled by what they read for the
    1 GiB device copy this script makes (d2d_copy_gbs), summed over the
    write/read kernels and divided by the number of steps in the run."""
    import csv
    import glob
    from collections import defaultdict

    vals = defaultdict(list)  # (kernel, counter) -> values per dispatch
    for d in args.counters_summary:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no *counter_collection.csv under {d}")
        for f in files:
            for row in csv.DictReader(open(f)):
                vals[(_short_kernel(row["Kernel_Name"]), row["Counter_Name"])].append(
                    float(row["Counter_Value"]))
    kernels = sorted({k for k, _ in vals})
    counters = sorted({c for _, c in vals})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for k in kernels:
        n = max(len(vals.get((k, c), [])) for c in counters)
        cells = []
        for c in counters:
            v = vals.get((k, c))
            cells.append(f"{sum(v) / len(v):.6g}" if v else "")
        print(f"| `{k}` | {n} | " + " | ".join(cells) + " |")
    if not {"FETCH_SIZE", "WRITE_SIZE"} <= set(counters):
        return
    copy = [k for k in kernels if "copyBuffer" in k]
    if not copy:
        sys.exit("no device-copy dispatch to calibrate FETCH_SIZE / WRITE_SIZE with")
    mean = lambda k, c: sum(vals[(k, c)]) / len(vals[(k, c)])
    fscale = 1048576.0 / mean(copy[0], "FETCH_SIZE")  # KiB per 1 GiB copy
    wscale = 1048576.0 / mean(copy[0], "WRITE_SIZE")
    schedule = "time-parallel" if args.variant in ("auto", "timepar") else "token-serial"
    if schedule == "time-parallel":
        # per-epoch launches (one read launch per epoch) or the fused
        # narrow-state kernel (one launch per step)
        rw = [k for k in kernels if k.startswith(("tp_read", "tp_update", "tp_fused"))]
        E = _epoch_len(wl, args.state)
        steps = (sum(len(vals[(k, "FETCH_SIZE")]) for k in rw if k.startswith("tp_read")) /
                 (-(-wl.T // E)) +
                 sum(len(vals[(k, "FETCH_SIZE")]) for k in rw if k.startswith("tp_fused")))
    else:
        rw = [k for k in kernels if k.startswith(("rw_serial_kernel", "rw_split_kernel"))]
        steps = sum(len(vals[(k, "FETCH_SIZE")]) for k in rw)
    fetch = sum(sum(vals[(k, "FETCH_SIZE")]) for k in rw) * 1024 * fscale / steps
    write = sum(sum(vals[(k, "WRITE_SIZE")]) for k in rw) * 1024 * wscale / steps
    tag = schedule.replace("-", "_") + "__" + wl.name.replace(" ", "_")
    if args.state != "f32":
        tag += f"__{args.state}_state"
    rec = {"schedule": schedule, "workload": wl.name, "kernels": rw,
           "hbm_bytes_per_step": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
           "fetch_scale": fscale, "write_scale": wscale, "steps_in_run": steps,
           "source_sha256": kernel_source_hash(schedule)}
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"\nFETCH_SIZE scale {fscale:.4f}, WRITE_SIZE scale {wscale:.4f} (1 GiB device copy); "
          f"write/read phase {fetch / 1e9:.2f} GB read + {write / 1e9:.2f} GB written = "
          f"{(fetch + write) / 1e9:.2f} GB per step over {steps:g} steps -> {path}")


def _epoch_len(wl, state="f32", cus=256):
    """Tokens per epoch of the time-parallel schedule (the library's rule:
    the largest power of two <= 4096 with E*W <= 2N and E*W <= 2^18, or
    with E*W <= N for a bfloat16 or E4M3 state and where chains x epochs
    would be fewer than a quarter of the `cus` compute units; for a
    bfloat16 or E4M3 state at most 256 where the one-launch kernel's
    (chain, 64-column slice) units fill the `cus` compute units; and no
    longer than the next power of two >= T)."""
    def for_cap(cap):
        e = 4096
        while e > 1 and (e * wl.W > (1 << 18) or e * wl.W > cap):
            e //= 2
        return e

    e = for_cap(2 * wl.N)
    if state != "f32" or 4 * wl.B * wl.H * -(-wl.T // e) < cus:
        e = for_cap(wl.N)
    units = wl.B * wl.H * -(-wl.d_v // 64)
    if state != "f32" and e > 256 and units >= cus and (units % cus == 0 or units >= 8 * cus):
        e = 256
    if e > wl.T:
        e = 1
        while e < wl.T:
            e *= 2
    return e


def _upload(d, dev):
    import numpy as np
    import torch

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    return {k: up(v) for k, v in d.items() if k != "src"}


def measure_forward(wl, d, dev, state, variant, steps, warmup):
    """Times `steps` whole forward steps (sdm_forward) after `warmup`, then
    the same number issued as sdm_prepare + sdm_apply with HIP events on the
    launch stream around each half.  Returns the figures of one workload."""
    import statistics

    import torch

    import sparse_memory_linear_select_amd as sdm

    dd = _upload(d, dev)
    st = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[state]
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[state]  # bytes per state element
    core = sdm.SDM(dd["M0"], wl.W, wl.R, state=st, state_scale_log2=FP8_SCALE_LOG2)
    B, T, H = wl.B, wl.T, wl.H
    y = torch.empty((B, T, H, wl.d_v), dtype=torch.float32, device=dev)
    M = torch.empty((B, H, wl.N, wl.d_v), dtype=st, device=dev)
    dt_code = sdm.BF16 if wl.dtype == "bf16" else sdm.F32
    ws_n = core.workspace_size(B, T, dt_code, variant)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    L = sdm.lib()
    stream = torch.cuda.current_stream(dev)
    sp = sdm._stream(dev)
    P = sdm._ptr

    def forward():
        sdm._check(L.sdm_forward(core._h, B, T, P(dd["kp"]), P(dd["qp"]), P(dd["v"]),
                                 P(dd["alpha"]), P(dd["beta"]), dt_code, variant, 0, P(ws), ws_n,
                                 P(y), P(M), sp))

    def prepare():
        sdm._check(L.sdm_prepare(core._h, B, T, P(dd["kp"]), P(dd["qp"]), P(dd["alpha"]),
                                 P(dd["beta"]), dt_code, variant, 0, P(ws), ws_n, P(M), sp))

    def apply():
        sdm._check(L.sdm_apply(core._h, B, T, P(dd["v"]), dt_code, variant, P(ws), ws_n, P(y),
                               P(M), sp))

    for _ in range(warmup):
        forward()
        prepare()
        apply()
    torch.cuda.synchronize()

    # timed region: `steps` whole steps (sdm_forward), an event after each
    ev_step = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev_step[0].record(stream)
    for i in range(steps):
        forward()
        ev_step[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev_step[0].elapsed_time(ev_step[-1]) / steps
    per_step = [ev_step[i].elapsed_time(ev_step[i + 1]) for i in range(steps)]

    # second pass: each step as sdm_prepare + sdm_apply on one stream, HIP
    # events bracketing the write/read kernels alone (roofline)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        prepare()
        e[1].record(stream)
        apply()
        e[2].record(stream)
    torch.cuda.synchronize()
    rw = [e[1].elapsed_time(e[2]) for e in ev]
    prep = [e[0].elapsed_time(e[1]) for e in ev]
    staged_ms = ev[0][0].elapsed_time(ev[-1][2]) / steps

    # third pass, the preparation split: sdm_prepare continuing the state (no
    # M <- M0) and sdm_select alone (the same selection, written in the API
    # layout instead of token records)
    Kw = torch.empty((B, T, H, wl.W), dtype=torch.float32, device=dev)
    Kr = torch.empty((B, T, H, wl.R), dtype=torch.float32, device=dev)
    Iw = torch.empty((B, T, H, wl.W), dtype=torch.int32, device=dev)
    Ir = torch.empty((B, T, H, wl.R), dtype=torch.int32, device=dev)

    def prepare_cont():
        sdm._check(L.sdm_prepare(core._h, B, T, P(dd["kp"]), P(dd["qp"]), P(dd["alpha"]),
                                 P(dd["beta"]), dt_code, variant, sdm.FLAG_CONTINUE, P(ws), ws_n,
                                 P(M), sp))

    def select():
        sdm._check(L.sdm_select(core._h, B, T, P(dd["kp"]), P(dd["qp"]), dt_code, P(Iw), P(Kw),
                                P(Ir), P(Kr), sp))

    ev3 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev3:
        e[0].record(stream)
        prepare_cont()
        e[1].record(stream)
        select()
        e[2].record(stream)
    torch.cuda.synchronize()
    prep_cont = sum(e[0].elapsed_time(e[1]) for e in ev3) / steps
    sel_ms = sum(e[1].elapsed_time(e[2]) for e in ev3) / steps
    del Kw, Kr, Iw, Ir
    rw_ms = sum(rw) / steps
    ht = wl.head_tokens
    row_bytes = ht * (2 * wl.W + wl.R) * wl.d_v * esz  # algorithmic row traffic per step
    schedule = sdm.variant_name(core, B, T, dt_code, variant)
    traffic = _traffic(wl, schedule, state)
    out = {
        "ms_per_step": ms_step, "ms_per_step_median": statistics.median(per_step),
        "head_tokens_per_s": ht / (ms_step * 1e-3),
        "staged_ms_per_step": staged_ms, "prepare_ms": sum(prep) / steps,
        "init_ms": sum(prep) / steps - prep_cont, "select_ms": sel_ms,
        "sort_plan_ms": prep_cont - sel_ms,
        "write_read_ms": rw_ms, "write_read_ms_median": statistics.median(rw),
        "schedule": schedule, "row_bytes": row_bytes, "wall_s_timed": wall,
        "effective_gbs": row_bytes / (rw_ms * 1e-3) / 1e9,
        "traffic": traffic,
        "hbm_gbs_counted": None if traffic is None else traffic / (rw_ms * 1e-3) / 1e9,
        "row_gbs_whole_step": row_bytes / (ms_step * 1e-3) / 1e9,
    }
    del dd, y, M, ws, core
    torch.cuda.empty_cache()
    return out


def _prepare_split(m):
    """init = prepare - prepare continuing the state (the marginal cost of
    M <- M0, which the selection carries where it can); select = sdm_select
    alone; sort + plan = the rest of the continuing prepare."""
    return {"init": m["init_ms"], "select": m["select_ms"], "sort + plan": m["sort_plan_ms"],
            "note": "init and sort + plan are differences of timed calls; select writes the "
                    "API layout rather than token records"}


def _workload_record(wl, m, cpu):
    """One workload's figures for the `workloads` object of the JSON line."""
    return {
        "config": {"B": wl.B, "T": wl.T, "H": wl.H, "sqrtN": wl.sqrtN, "d_v": wl.d_v, "W": wl.W,
                   "R": wl.R, "inputs": wl.dtype, "key_reuse": wl.reuse},
        "schedule": m["schedule"],
        "head_tokens_per_s": m["head_tokens_per_s"], "ms_per_step": m["ms_per_step"],
        "ms_per_step_median": m["ms_per_step_median"], "prepare_ms": m["prepare_ms"],
        "prepare_split_ms": _prepare_split(m),
        "write_read_ms": m["write_read_ms"], "algorithmic_row_bytes": m["row_bytes"],
        "effective_gbs": m["effective_gbs"], "frac": m["effective_gbs"] / PEAK_HBM_GBS,
        "traffic": m["traffic"], "hbm_gbs_counted": m["hbm_gbs_counted"],
        "frac_counted": (None if m["hbm_gbs_counted"] is None
                         else m["hbm_gbs_counted"] / PEAK_HBM_GBS),
        "frac_whole_step": m["row_gbs_whole_step"] / PEAK_HBM_GBS,
        "cpu_baseline": cpu,
    }


# bounded oracle samples per workload: (sequences, tokens, runs)
CPU_SAMPLES = {0: (1, None, 5), 1: (2, None, 5), 2: (1, 4096, 3), 3: (1, 4096, 3),
               4: (1, 16384, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=1,
                    help="synthetic workload index (default 1: the 1.4B-style layer)")
    ap.add_argument("--variant", choices=["auto", "serial", "timepar"], default="auto",
                    help="write/read schedule (default: the library's choice)")
    ap.add_argument("--state", choices=["f32", "bf16", "fp8"], default="f32",
                    help="element type of the state M (bf16, or fp8: E4M3 codes scaled by "
                         f"2^{FP8_SCALE_LOG2})")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure the headline workload only (no `workloads` object)")
    ap.add_argument("--decode", action="store_true",
                    help="measure one-token decode steps (continuing the state) instead")
    ap.add_argument("--backward", action="store_true",
                    help="measure the backward (sdm_backward: forward recompute + reverse) instead")
    ap.add_argument("--backward-chunks", type=int, default=0,
                    help="backward workspace sized for this many chunks of epochs (0: the least "
                         "memory; 1: the whole sequence at once)")
    ap.add_argument("--counters-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 CSV output directories instead of running "
                         "(see counters_summary)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the SDM core shards by (sequence, head) chain or by "
              "column with no exchange on the hot path, so only --gpus 1 is run here",
              file=sys.stderr)
        sys.exit(2)

    import sdm_inputs as si

    if args.counters_summary:
        return counters_summary(args, si.WORKLOADS[args.workload])

    import torch

    import sparse_memory_linear_select_amd as sdm

    wl = si.WORKLOADS[args.workload]
    if args.decode:
        return decode(args, wl)
    if args.backward:
        return backward(args, wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    var = {"auto": sdm.AUTO, "serial": sdm.SERIAL, "timepar": sdm.TIMEPAR}[args.variant]

    _log(f"workload {args.workload}: {wl}")
    t = time.perf_counter()
    d = si.generate(wl)
    _log(f"inputs generated in {time.perf_counter() - t:.1f}s")
    m = measure_forward(wl, d, dev, args.state, var, args.steps, args.warmup)
    _log(f"headline: {m['ms_per_step']:.3f} ms/step, write/read {m['write_read_ms']:.3f} ms")
    copy_gbs = d2d_copy_gbs(dev)

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        seqs, T, runs = CPU_SAMPLES.get(args.workload, (1, 1024, 3))
        cpu = cpu_baseline(d, wl, seqs, T, args.state, runs=runs)
        # one host core: the tiny workload whole, and a slice of this one
        cpu1 = {"tiny": cpu_baseline(si.generate(si.WORKLOADS[0]), si.WORKLOADS[0], 1,
                                     state=args.state, threads=1, runs=5)}
        if args.workload != 0:
            cpu1[wl.name] = cpu_baseline(d, wl, 1, min(wl.T, 1024), args.state, threads=1, runs=3)
    del d

    dec = None
    if not args.no_workloads and args.variant == "auto" and args.state == "f32":
        _log("decode steps")
        r = measure_decode(wl, 200, 10)
        dec = {"workload": wl.name, "B": wl.B, "eager_us_per_step": r["us_per_step"],
               "graph_replay_us_per_step": r["graph_replay_us_per_step"],
               "steps": r["steps"], "prefill_tokens": r["prefill_tokens"],
               "note": "one token for each of B sequences per call, state continued; "
                       "sdm_forward with T = 1 (one launch)"}
        _log(f"  {r['graph_replay_us_per_step']:.2f} us/step replayed, "
             f"{r['us_per_step']:.2f} us/step eager")

    workloads = {}
    if not args.no_workloads and args.variant == "auto" and args.state == "f32":
        for c in (1, 2, 3, 4):
            if c == args.workload:
                continue
            w = si.WORKLOADS[c]
            _log(f"workload {c}: {w}")
            t = time.perf_counter()
            dw = si.generate(w)
            _log(f"  inputs generated in {time.perf_counter() - t:.1f}s")
            mw = measure_forward(w, dw, dev, "f32", sdm.AUTO, min(args.steps, 5), 1)
            _log(f"  {mw['ms_per_step']:.3f} ms/step, write/read {mw['write_read_ms']:.3f} ms")
            cw = None
            if not args.no_cpu_baseline:
                seqs, T, runs = CPU_SAMPLES[c]
                cw = cpu_baseline(dw, w, seqs, T, "f32", runs=runs)
            del dw
            workloads[w.name] = _workload_record(w, mw, cw)

    out = {
        "metric": METRIC,
        "value": m["head_tokens_per_s"],
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {("f32", "f32"): "f32", ("bf16", "f32"): "bf16 inputs, f32 state",
                  ("f32", "bf16"): "f32 compute, bf16 state",
                  ("bf16", "bf16"): "bf16 inputs, f32 compute, bf16 state",
                  ("f32", "fp8"): "f32 compute, fp8 (E4M3) state",
                  ("bf16", "fp8"): "bf16 inputs, f32 compute, fp8 (E4M3) state"}[
                      (wl.dtype, args.state)],
        "data": "synthetic (seeded; recipe in sdm_inputs.py)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "sqrtN": wl.sqrtN,
                   "N": wl.N, "d_v": wl.d_v, "W": wl.W, "R": wl.R, "inputs": wl.dtype,
                   "state": args.state, "schedule": m["schedule"]},
        "ms_per_step_median": m["ms_per_step_median"],
        "row_gbs_whole_step": m["row_gbs_whole_step"],
        "breakdown_ms": {"staged step (prepare + apply, one stream)": m["staged_ms_per_step"],
                         "prepare (init+select+sort+plan)": m["prepare_ms"],
                         "prepare split": _prepare_split(m),
                         "write+read": m["write_read_ms"],
                         "write+read median": m["write_read_ms_median"]},
        "wall_s_timed": m["wall_s_timed"],
        "roofline": {"bound": "hbm", "achieved": m["effective_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": m["effective_gbs"] / PEAK_HBM_GBS,
                     "traffic": m["traffic"],
                     "traffic_unit": "HBM bytes per step (write/read phase, counters)",
                     "kernel": rw_kernels(m["schedule"], args.state),
                     "timing": "write/read kernels bracketed by HIP events on their stream in "
                               "a second pass of K steps issued as sdm_prepare + sdm_apply",
                     "achieved_is": "effective: algorithmic row bytes ((2W+R) d_v per "
                                    "head-token) / write-read time; repeated writes to a slot "
                                    "within an epoch merge, so HBM moves fewer bytes",
                     "algorithmic_bytes": m["row_bytes"],
                     "hbm_gbs_counted": m["hbm_gbs_counted"],
                     "frac_counted": (None if m["hbm_gbs_counted"] is None
                                      else m["hbm_gbs_counted"] / PEAK_HBM_GBS),
                     "frac_whole_step": m["row_gbs_whole_step"] / PEAK_HBM_GBS,
                     "d2d_copy_gbs": copy_gbs,
                     "frac_of_copy": m["effective_gbs"] / copy_gbs},
        "cpu_baseline": cpu,
        "cpu_baseline_1core": cpu1,
        "workloads": workloads or None,
        "decode": dec,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
