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
METRIC = "SDM select+write+read head-tokens/s and achieved HBM GB/s (% peak)"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


SCHEDULES = {  # schedule -> (kernel source, kernels of the write/read phase)
    "token-serial": ("rw_serial.hip", "rw_serial_kernel (one launch)"),
    "time-parallel": ("rw_timepar.hip", "tp_read_kernel + tp_update_kernel (one pair per epoch)"),
}


def _traffic(wl, schedule, state="f32"):
    """Counter-measured HBM bytes of the write/read phase per step, if a
    committed summary exists for this workload, schedule and state type and
    the kernel source is unchanged since the counters were taken; else None."""
    src_name = SCHEDULES[schedule][0]
    tag = schedule.replace("-", "_") + "__" + wl.name.replace(" ", "_")
    if state != "f32":
        tag += f"__{state}_state"
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, "sparse_memory_linear_select_amd", "csrc", src_name),
                   "rb").read()
        if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
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


def cpu_baseline(d, wl, seqs, state="f32"):
    """The float64 oracle on the first `seqs` sequences of the same inputs."""
    import oracle

    sub = {k: (v[:seqs] if k not in ("M0",) else v) for k, v in d.items() if k != "src"}
    cores = oracle.default_threads()
    t = time.perf_counter()
    oracle.forward(sub, wl.sqrtN, wl.W, wl.R, threads=cores, state=state)
    dt = time.perf_counter() - t
    ht = seqs * wl.T * wl.H
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": ht / dt, "unit": "head-tokens/s", "cores": cores, "kind": "oracle",
            "cpu": model,
            "sample": f"{seqs} of {wl.B} sequences of the workload ({ht} head-tokens, all "
                      f"{wl.d_v} columns), select + init + recurrence, {dt:.2f} s wall"}


def decode(args, wl):
    """Decode: B sequences advance by one token per call (T = 1), continuing
    from the state left by a 256-token prefill.  Reports the step latency."""
    import numpy as np
    import torch

    import sdm_inputs as si
    import sparse_memory_linear_select_amd as sdm

    prefix, steps, warm = 256, args.steps * 20, args.warmup * 5
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
    var = {"auto": sdm.AUTO, "serial": sdm.SERIAL, "timepar": sdm.TIMEPAR}[args.variant]
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
    print(json.dumps({
        "metric": "SDM decode step latency (one token for each of B sequences, state continued)",
        "value": us, "unit": "us/step", "higher_is_better": False, "n_gpus": 1, "steps": steps,
        "warmup": warm, "head_tokens_per_s": wl.B * wl.H / (us * 1e-6),
        "graph_replay_us_per_step": us_graph,
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "sqrtN": wl.sqrtN, "d_v": wl.d_v,
                   "W": wl.W, "R": wl.R, "prefill_tokens": prefix,
                   "schedule": sdm.variant_name(core, wl.B, 1, dt_code, var)},
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


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=1,
                    help="synthetic workload index (default 1: the 1.4B-style layer)")
    ap.add_argument("--cpu-seqs", type=int, default=None,
                    help="sequences in the CPU-baseline sample (default: all)")
    ap.add_argument("--variant", choices=["auto", "serial", "timepar"], default="auto",
                    help="write/read schedule (default: the library's choice)")
    ap.add_argument("--state", choices=["f32", "bf16"], default="f32",
                    help="element type of the state M (bf16: reduced-precision state)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="measure one-token decode steps (continuing the state) instead")
    ap.add_argument("--backward", action="store_true",
                    help="measure the backward (sdm_backward: forward recompute + reverse) instead")
    ap.add_argument("--backward-chunks", type=int, default=0,
                    help="backward workspace sized for this many chunks of epochs (0: the least "
                         "memory; 1: the whole sequence at once)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the SDM core shards by (sequence, head) chain or by "
              "column with no exchange on the hot path, so only --gpus 1 is run here",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sdm_inputs as si
    import sparse_memory_linear_select_amd as sdm

    wl = si.WORKLOADS[args.workload]
    if args.decode:
        return decode(args, wl)
    if args.backward:
        return backward(args, wl)
    _log(f"workload {args.workload}: {wl}")
    t = time.perf_counter()
    d = si.generate(wl)
    _log(f"inputs generated in {time.perf_counter() - t:.1f}s")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        import numpy as np
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    dd = {k: up(v) for k, v in d.items() if k != "src"}
    state = torch.bfloat16 if args.state == "bf16" else torch.float32
    esz = 2 if args.state == "bf16" else 4  # bytes per state element
    core = sdm.SDM(dd["M0"], wl.W, wl.R, state=state)
    B, T, H = wl.B, wl.T, wl.H
    y = torch.empty((B, T, H, wl.d_v), dtype=torch.float32, device=dev)
    M = torch.empty((B, H, wl.N, wl.d_v), dtype=state, device=dev)
    dt_code = sdm.BF16 if wl.dtype == "bf16" else sdm.F32
    var = {"auto": sdm.AUTO, "serial": sdm.SERIAL, "timepar": sdm.TIMEPAR}[args.variant]
    ws_n = core.workspace_size(B, T, dt_code, var)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    L = sdm.lib()
    stream = torch.cuda.current_stream(dev)
    sp = sdm._stream(dev)
    P = sdm._ptr

    def forward():
        sdm._check(L.sdm_forward(core._h, B, T, P(dd["kp"]), P(dd["qp"]), P(dd["v"]),
                                 P(dd["alpha"]), P(dd["beta"]), dt_code, var, 0, P(ws), ws_n,
                                 P(y), P(M), sp))

    def prepare():
        sdm._check(L.sdm_prepare(core._h, B, T, P(dd["kp"]), P(dd["qp"]), P(dd["alpha"]),
                                 P(dd["beta"]), dt_code, var, 0, P(ws), ws_n, P(M), sp))

    def apply():
        sdm._check(L.sdm_apply(core._h, B, T, P(dd["v"]), dt_code, var, P(ws), ws_n, P(y),
                               P(M), sp))

    for _ in range(args.warmup):
        forward()
        prepare()
        apply()
    torch.cuda.synchronize()

    # timed region: K whole steps (sdm_forward)
    t0_ev, t1_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0_ev.record(stream)
    for _ in range(args.steps):
        forward()
    t1_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0_ev.elapsed_time(t1_ev) / args.steps

    # second pass, K steps issued as sdm_prepare + sdm_apply on one stream, so
    # that HIP events bracket the write/read kernels alone (roofline)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        prepare()
        e[1].record(stream)
        apply()
        e[2].record(stream)
    torch.cuda.synchronize()
    staged_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    rw_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    ht = wl.head_tokens
    row_bytes = ht * (2 * wl.W + wl.R) * wl.d_v * esz  # algorithmic row traffic per step
    achieved = row_bytes / (rw_ms * 1e-3) / 1e9
    schedule = sdm.variant_name(core, B, T, dt_code, var)
    traffic = _traffic(wl, schedule, args.state)

    copy_gbs = d2d_copy_gbs(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, wl, args.cpu_seqs or wl.B, args.state)

    out = {
        "metric": METRIC,
        "value": ht / (ms_step * 1e-3),
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {("f32", "f32"): "f32", ("bf16", "f32"): "bf16 inputs, f32 state",
                  ("f32", "bf16"): "f32 compute, bf16 state",
                  ("bf16", "bf16"): "bf16 inputs, f32 compute, bf16 state"}[(wl.dtype, args.state)],
        "data": "synthetic (seeded; recipe in sdm_inputs.py)",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "sqrtN": wl.sqrtN, "N": wl.N,
                   "d_v": wl.d_v, "W": wl.W, "R": wl.R, "inputs": wl.dtype,
                   "state": args.state, "schedule": schedule},
        "row_gbs_whole_step": row_bytes / (ms_step * 1e-3) / 1e9,
        "breakdown_ms": {"staged step (prepare + apply, one stream)": staged_ms,
                         "prepare (init+select+plan/sort)": prep_ms, "write+read": rw_ms},
        "wall_s_timed": wall,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per step (write/read phase, counters)",
                     "kernel": SCHEDULES[schedule][1],
                     "timing": "write/read kernels bracketed by HIP events on their stream in "
                               "a second pass of K steps issued as sdm_prepare + sdm_apply",
                     "algorithmic_bytes": row_bytes,
                     "d2d_copy_gbs": copy_gbs,
                     "frac_of_copy": achieved / copy_gbs},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
