#!/usr/bin/env python3
"""Benchmark of the multi-head LSTM forward hot path on one MI355X.

A step is one whole forward pass of the workload through the C ABI's fused
entry point (rnn_fwd_lstm / rnn_fwd_gru: input projection as a bf16 MFMA
contraction over all T*B rows, then the sequential recurrence with R
resident; the two overlap when the recurrence leaves half the chip free),
plus rnn_bwd_lstm for the forward+backward workload, on synthetic inputs
already resident in HBM.  `value` is recurrent TFLOP/s: the algorithmic
flops of the recurrent products (2*B*H*G*Dh per step, the block-diagonal R
only; twice that with the backward) divided by the wall time of the step,
K steps back to back with nothing else on the stream between them.  K more
steps with HIP events around each phase then give the per-phase figures.

The roofline entry is for the dominant kernel, the recurrence: after the
timed steps, min(K, 20) more launches of the recurrence alone (rnn_rec_lstm
on the projection's output) are bracketed one by one with HIP events on the
stream they run on, and its average launch duration gives `achieved`.  The
input projection alone is timed the same way.

Prints ONE JSON line (see the keys below).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-clock]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import shutil
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "recurrent TFLOP/s and time-steps/s, multi-head LSTM fwd B=16 NH=6 Dh=128"
HEADLINE = "lstm_mh_b16_nh6_dh128"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
NUM_CU = 256
CU_BF16_TFLOPS = PEAK_BF16_TFLOPS / NUM_CU
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# launches of the recurrence alone and of the projection alone, each timed
KERNEL_LAUNCHES = 20
KERNEL_SOURCES = [os.path.join(ROOT, "gru_recurrence_amd", "csrc", f)
                  for f in ("rec_fwd.hip", "gates.h", "common.h")]
KERNEL_ARGS_HEADER = os.path.join(ROOT, "gru_recurrence_amd", "csrc", "kernels.h")


def kernel_source_hash() -> str:
    """Hash of what the recurrence kernel is compiled from: its source file,
    the device helpers it includes and its argument block (struct RecArgs);
    other declarations in the kernels header do not change its code."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    with open(KERNEL_ARGS_HEADER) as f:
        hdr = f.read()
    i = hdr.index("struct RecArgs {")
    h.update(hdr[i:hdr.index("};", i) + 2].encode())
    return h.hexdigest()[:16]


def recurrent_flops(w: synth.Workload, T=None) -> float:
    d = w.dims
    G = synth.gates_of(w.cell)
    return 2.0 * d.B * d.NH * d.Dh * G * d.Dh * (T if T is not None else d.T)


def rec_kernel_name(w: synth.Workload, plan: str) -> str:
    """Name of the recurrence kernel the plan launches, as the profiler shows
    it (template arguments: cell, Dh, cell update passes, steps per group,
    waits, rows in lane groups)."""
    if "multi_cu" in plan:
        return "rec_fwd_mc_kernel"
    if "split_R" in plan:
        return "rec_fwd_wide_kernel<%d>" % (0 if w.cell == "lstm" else 1)
    if "mfma" not in plan:
        return "rec_fwd_simple_kernel"
    passes = int(plan.split("units_per_thread=")[1].split()[0])
    rows = int(plan.split("rows_per_wg=")[1].split()[0])
    lanes = 1 < rows <= 8
    one = {("lstm", 128): 2, ("gru", 64): 16}.get((w.cell, w.dims.Dh), 8)
    pd = {1: one if rows == 1 else 4, 2: 2, 4: 2}[passes]
    return "rec_fwd_mfma_kernel<%d, %d, %d, %d, false, %s>" % (
        0 if w.cell == "lstm" else 1, w.dims.Dh, passes, pd, "true" if lanes else "false")


def gfx_clock_under_load(step, torch) -> float | None:
    """GFX clock (MHz; mean over the XCDs and over two readings) as amd-smi
    reports it while the workload's step runs in a loop, the first reading
    after one second of it (amd-smi's figures lag the load); None where
    amd-smi is missing or its output cannot be read.  The recurrence is bound
    by its per-step latency, which scales with this clock."""
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    res = {"v": []}

    def read():
        r = subprocess.run([exe, "metric", "-g", "0", "--clock", "--json"],
                           capture_output=True, text=True, timeout=20)
        clk = json.loads(r.stdout)["gpu_data"][0]["clock"]
        v = [c["clk"]["value"] for k, c in clk.items()
             if k.startswith("gfx_") and isinstance(c, dict) and isinstance(c.get("clk"), dict)
             and isinstance(c["clk"].get("value"), (int, float))]
        if v:
            res["v"].append(sum(v) / len(v))

    def sample():
        try:
            time.sleep(1.0)
            read()
            time.sleep(0.5)
            read()
        except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
            pass

    th = threading.Thread(target=sample)
    th.start()
    while th.is_alive():
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    th.join()
    return round(sum(res["v"]) / len(res["v"]), 1) if res["v"] else None


def traffic_per_launch():
    """HBM bytes per recurrence launch from committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ONE_CORE = r"""
import sys, time
sys.path.insert(0, %r)
import oracle, synth
w = synth.WORKLOADS[%r]
d = w.dims
c = synth.workload_case(w, synth.Dims(%d, d.B, d.Din, d.NH, d.Dh))
args = (c.f64("x"), c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"), c.f64("c0"))
oracle.lstm_fwd(*args, NH=d.NH, Dh=d.Dh)
best = 1e30
for _ in range(3):
    t0 = time.perf_counter()
    oracle.lstm_fwd(*args, NH=d.NH, Dh=d.Dh)
    best = min(best, time.perf_counter() - t0)
print(oracle.num_threads(), best)
"""


def cpu_one_core(w: synth.Workload, Tp: int = 64):
    """The oracle on one core (OMP_NUM_THREADS=1, a child process) over the
    first Tp steps of the workload, all chains; returns (seconds, threads)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    out = subprocess.run([sys.executable, "-c", _ONE_CORE % (ROOT, w.name, Tp)], env=env,
                         capture_output=True, text=True, timeout=600)
    thr, sec = out.stdout.split()[-2:]
    return float(sec), int(thr)


def cpu_baseline(w: synth.Workload, c, budget_s: float):
    """Time the oracle (double-precision scalar C, OpenMP over independent
    chains) on a T-prefix of the same workload, all chains, and express it in
    the metric's unit (recurrent TFLOP/s of the whole forward).  Also on one
    core over the first 64 steps, scaled to T (the work is linear in T)."""
    import oracle
    d = w.dims
    # one short probe to size the sample to ~budget_s of CPU work
    Tp = 8
    x = c.f64("x")
    args = (c.f64("W"), c.f64("R"), c.f64("b"), c.f64("h0"), c.f64("c0"))
    t0 = time.perf_counter()
    oracle.lstm_fwd(x[:Tp], *args, NH=d.NH, Dh=d.Dh)
    probe = time.perf_counter() - t0
    Ts = int(min(d.T, max(Tp, Tp * budget_s / max(probe, 1e-6))))
    reps, el = 0, 0.0
    while reps == 0 or (el < 0.5 * budget_s and reps < 20):
        t0 = time.perf_counter()
        oracle.lstm_fwd(x[:Ts], *args, NH=d.NH, Dh=d.Dh)
        el += time.perf_counter() - t0
        reps += 1
    per = el / reps
    flops = recurrent_flops(w, Ts)
    out = {"value": flops / per / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": "whole forward (input projection + recurrence) of the first %d of %d "
                     "steps, all %d chains, float64; mean of %d runs, %.3f s each"
                     % (Ts, d.T, d.B * d.NH, reps, per),
           "time_steps_per_s": Ts / per}
    try:
        sec, thr = cpu_one_core(w, 64)
        out["one_core"] = {"threads": thr, "sample": "first 64 steps, all chains, best of 3",
                           "seconds": round(sec, 4),
                           "scaled_to_T_seconds": round(sec * d.T / 64, 3),
                           "value_scaled": recurrent_flops(w, 64) / sec / 1e12,
                           "note": "scaled: 64-step time x T/64"}
    except Exception as e:  # the all-core figure above stands on its own
        out["one_core"] = {"error": str(e)[:200]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock reading under load (a loop of steps; profiles use this)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times) and exit; "
                         "used to scale the HBM byte counters of a profiler run")
    args = ap.parse_args()

    if args.copy_calibration_mb > 0:
        import torch
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_mb": args.copy_calibration_mb,
                          "bytes_read_per_copy": 4 * n, "bytes_written_per_copy": 4 * n}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; the recurrence shards by heads or "
              "batch rows with no exchange, but no multi-GPU path is built "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gru_recurrence_amd as g

    w = synth.WORKLOADS[args.workload]
    d = w.dims
    stacked = w.layers > 1
    cs = synth.workload_stack_case(w) if stacked else [synth.workload_case(w)]
    c = cs[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(name):
        if name in c.bits:
            return torch.from_numpy(c.bits[name].view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(c.vals[name])).to(dev)

    lstm = w.cell == "lstm"
    G = 4 if lstm else 3
    x, W, R, b = to_dev("x"), to_dev("W"), to_dev("R"), to_dev("b")
    h0 = to_dev("h0")
    c0 = to_dev("c0") if lstm else None
    H, N = d.NH * d.Dh, d.NH * G * d.Dh
    f32 = torch.float32
    gx = torch.empty((d.T, d.B, N), dtype=f32, device=dev)
    outs = dict(h_seq=torch.empty((d.T, d.B, H), dtype=f32, device=dev),
                c_seq=torch.empty((d.T, d.B, H), dtype=f32, device=dev),
                hT=torch.empty((d.B, H), dtype=f32, device=dev),
                cT=torch.empty((d.B, H), dtype=f32, device=dev))
    dims = g.dims_of(x, R)
    dtc = g.RNN_BF16 if w.dtype == "bf16" else g.RNN_F32
    op = g.OP_REC_LSTM if lstm else g.OP_REC_GRU
    ws = torch.empty(g.workspace_size(op, dims, dtc), dtype=torch.uint8, device=dev)
    plan = g.plan_describe(op, dims, dtc)
    stream = torch.cuda.current_stream()

    backward = w.backward
    if backward:
        dH = to_dev("dH")
        ws_b = torch.empty(g.workspace_size(g.OP_BWD_LSTM, dims, dtc), dtype=torch.uint8, device=dev)
        grads = dict(dx=torch.empty((d.T, d.B, d.Din), dtype=f32, device=dev),
                     dW=torch.empty((d.Din, N), dtype=f32, device=dev),
                     dR=torch.empty((d.NH, d.Dh, 4 * d.Dh), dtype=f32, device=dev),
                     db=torch.empty((N,), dtype=f32, device=dev),
                     dh0=torch.empty((d.B, H), dtype=f32, device=dev),
                     dc0=torch.empty((d.B, H), dtype=f32, device=dev))

    fop = g.OP_FWD_LSTM if lstm else g.OP_FWD_GRU
    ws_f = torch.empty(g.workspace_size(fop, dims, dtc), dtype=torch.uint8, device=dev)
    fplan = g.plan_describe(fop, dims, dtc)
    if stacked:
        # every layer's weights; layer 0 takes x, layer l > 0 the h of layer l-1
        def layer_dev(ci, name):
            if name in ci.bits:
                return torch.from_numpy(ci.bits[name].view(np.int16).copy()).view(
                    torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(ci.vals[name])).to(dev)
        L = w.layers
        Ws = [layer_dev(ci, "W") for ci in cs]
        Rs = [layer_dev(ci, "R") for ci in cs]
        bs = [layer_dev(ci, "b") for ci in cs]
        h0s = torch.stack([layer_dev(ci, "h0") for ci in cs])
        c0s = torch.stack([layer_dev(ci, "c0") for ci in cs]) if lstm else None
        outs_s = dict(h_seq=outs["h_seq"], c_seq=outs["c_seq"],
                      hT=torch.empty((L, d.B, H), dtype=f32, device=dev),
                      cT=torch.empty((L, d.B, H), dtype=f32, device=dev))
        ws_f = torch.empty(g.workspace_size_stack(fop, dims, L, dtc), dtype=torch.uint8,
                           device=dev)

    chunked = w.chunk > 0
    if chunked:
        # the forward in chunks (checkpoints at the chunk ends when the
        # backward follows, which then recomputes each segment from them)
        ws_f = torch.empty(g.workspace_size_chunked(fop, dims, w.chunk, dtc), dtype=torch.uint8,
                           device=dev)
        nck = (d.T + w.chunk - 1) // w.chunk
        outs_c = dict(outs)
        if backward:
            outs_c["h_ckpt"] = torch.empty((nck, d.B, H), dtype=f32, device=dev)
            outs_c["c_ckpt"] = torch.empty((nck, d.B, H), dtype=f32, device=dev)
            ws_b = torch.empty(g.workspace_size_chunked(g.OP_BWD_LSTM, dims, w.chunk, dtc),
                               dtype=torch.uint8, device=dev)

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if chunked:
            g.lstm_fwd_chunked(x, W, R, b, h0, c0, chunk=w.chunk, with_seq=not backward,
                               ckpt=backward, ws=ws_f, out=outs_c, stream=stream)
            if evs is not None:
                evs[1].record(stream)
            if backward:
                g.lstm_bwd_ckpt(x, W, R, b, h0, c0, outs_c["h_ckpt"], outs_c["c_ckpt"], dH,
                                chunk=w.chunk, ws=ws_b, out=grads, stream=stream)
                if evs is not None:
                    evs[2].record(stream)
            return
        if stacked and lstm:
            g.lstm_stack_fwd(x, Ws, Rs, bs, h0s, c0s, ws=ws_f, out=outs_s, stream=stream)
        elif stacked:
            g.gru_stack_fwd(x, Ws, Rs, bs, h0s, ws=ws_f, out=outs_s, stream=stream)
        elif lstm:
            g.lstm_fwd(x, W, R, b, h0, c0, ws=ws_f, out=outs, stream=stream)
        else:
            g.gru_fwd(x, W, R, b, h0, ws=ws_f, out=outs, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        if backward:
            g.lstm_bwd(x, W, R, b, h0, c0, outs["h_seq"], outs["c_seq"], dH, ws=ws_b,
                       out=grads, stream=stream)
            if evs is not None:
                evs[2].record(stream)

    def timed(fn, n):
        """n calls of fn, each bracketed by events on `stream`; (mean, median,
        min) ms."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        return float(np.mean(ms)), float(np.median(ms)), float(np.min(ms))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps back to back, nothing else on the stream between them
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # then as many steps again with events around each phase, for the
    # per-phase figures (the events themselves take a few microseconds of
    # stream time per step, which is why the timed loop above has none)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2 if backward else 1]) for e in evs]
    for wsx in (ws_f,) + ((ws_b,) if backward else ()):
        st = g.workspace_status(wsx, stream)
        if st != g.RNN_OK:
            print("bench.py: kernel reported %s" % g.status_str(st), file=sys.stderr)
            sys.exit(1)

    # the two kernels of the forward, each on its own (the forward stages W
    # transposed and runs the k-major contraction; here W^T is made once)
    if dtc == g.RNN_BF16 and d.Din % 32 == 0:
        Wt = W.t().contiguous()

        def proj():
            g.input_proj_t(x, Wt, b, out=gx, stream=stream)
    else:
        def proj():
            g.input_proj(x, W, b, out=gx, stream=stream)

    def rec():
        if lstm:
            g.rec_lstm(gx, R, h0, c0, ws=ws, out=outs, stream=stream)
        else:
            g.rec_gru(gx, R, h0, ws=ws, out=outs, stream=stream)

    proj()
    rec()
    # each kernel alone: a fixed count of launches (a long run of the
    # projection alone at 1.3-1.4 kW lowers the clock it runs at)
    nk = min(args.steps, KERNEL_LAUNCHES)
    proj_avg, proj_med, proj_min = timed(proj, nk)
    rec_avg, rec_med, rec_min = timed(rec, nk)
    clock = None if args.no_clock else gfx_clock_under_load(step, torch)
    st = g.workspace_status(ws, stream)
    if st != g.RNN_OK:
        print("bench.py: kernel reported %s" % g.status_str(st), file=sys.stderr)
        sys.exit(1)

    ms_step = 1e3 * wall / args.steps
    # forward + backward: the reverse sweep's dA R^T products add the same
    # recurrent flops again
    rflops = recurrent_flops(w) * (2 if backward else 1) * w.layers
    value = rflops / (ms_step * 1e-3) / 1e12
    achieved = recurrent_flops(w) / (rec_avg * 1e-3) / 1e12
    gemm_flops = 2.0 * d.T * d.B * d.Din * N
    ncu_engaged = int(plan.split(" wg=")[1].split()[0])
    cands, best = g.plan_search(op, dims, dtc)
    predicted = float(plan.split("predicted_ns_per_step=")[1].split()[0])
    out = {
        "metric": METRIC if args.workload == HEADLINE else METRIC.split(",")[0] + ", " + w.name,
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller, bf16 RNE), random-init weights",
        "config": {"workload": w.name, "cell": w.cell, "T": d.T, "B": d.B, "NH": d.NH,
                   "Dh": d.Dh, "Din": d.Din, "hidden": H, "layers": w.layers,
                   "parallelism": "single GPU"},
        "time_steps_per_s": round(d.T / (ms_step * 1e-3), 1),
        "forward_call": {"avg_ms": round(float(np.mean(fwd_ms)), 4), "plan": fplan},
        "step_event_ms": {"median": round(float(np.median(step_ms)), 4),
                          "min": round(float(np.min(step_ms)), 4)},
        "gfx_clock_mhz_under_load": clock,
        "recurrence": {"avg_launch_ms": round(rec_avg, 4), "median_launch_ms": round(rec_med, 4),
                       "min_launch_ms": round(rec_min, 4), "tflops": round(achieved, 3),
                       "ns_per_time_step": round(rec_avg * 1e6 / d.T, 1),
                       "time_steps_per_s": round(d.T / (rec_avg * 1e-3), 1),
                       "engaged_cus": ncu_engaged,
                       "engaged_cu_peak_tflops": round(ncu_engaged * CU_BF16_TFLOPS, 1),
                       "frac_of_engaged_cu_peak": round(achieved / (ncu_engaged * CU_BF16_TFLOPS), 4),
                       "plan": plan,
                       "plan_search": {"candidates": len(cands),
                                       "feasible": sum(1 for c in cands if c["feasible"]),
                                       "predicted_ns_per_step": predicted,
                                       "measured_ns_per_step": round(rec_avg * 1e6 / d.T, 1)}},
        "input_projection": {"avg_launch_ms": round(proj_avg, 4),
                             "median_launch_ms": round(proj_med, 4),
                             "min_launch_ms": round(proj_min, 4),
                             "tflops": round(gemm_flops / (proj_avg * 1e-3) / 1e12, 2),
                             "frac_of_peak": round(gemm_flops / (proj_avg * 1e-3) / 1e12
                                                   / PEAK_BF16_TFLOPS, 4)},
        # the recurrence is bound by the latency of its per-step dependency
        # chain (one live batch row per MFMA, a barrier per step), not by the
        # chip's MFMA throughput or HBM: `frac` is against the bf16 MFMA peak
        "roofline": {"kernel": rec_kernel_name(w, plan), "bound": "latency",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 5),
                     "traffic": traffic_per_launch()},
        # the whole forward call (projection and recurrence, one launch where
        # they overlap): all its flops over its average call time
        "forward_call_roofline": {
            "achieved": round((gemm_flops + recurrent_flops(w)) / (float(np.mean(fwd_ms)) * 1e-3)
                              / 1e12, 3),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round((gemm_flops + recurrent_flops(w)) / (float(np.mean(fwd_ms)) * 1e-3)
                          / 1e12 / PEAK_BF16_TFLOPS, 5)},
        "cpu_baseline": None,
    }
    if backward:
        bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
        out["backward"] = {"avg_call_ms": round(float(np.mean(bwd_ms)), 4),
                           "note": "rnn_bwd_lstm: recompute GEMMs, reverse sweep in time chunks "
                                   "with each chunk's dx/dW/dR GEMMs beside the next chunk's sweep"}
    if chunked:
        out["config"]["chunk"] = w.chunk
        out["workspace_bytes"] = {
            "forward_chunked": int(ws_f.numel()),
            "forward_one_piece": int(g.workspace_size(fop, dims, dtc))}
        if backward:
            out["workspace_bytes"]["backward_checkpointed"] = int(ws_b.numel())
            out["workspace_bytes"]["backward_one_piece"] = int(
                g.workspace_size(g.OP_BWD_LSTM, dims, dtc))
            out["backward"]["note"] = ("rnn_bwd_lstm_ckpt: per segment of %d steps, the forward "
                                       "recomputed from the checkpoint, then BPTT" % w.chunk)
        out["forward_call"]["note"] = ("rnn_fwd_lstm_chunked in chunks of %d steps; the recurrence "
                                       "and input projection entries time one-piece kernels"
                                       % w.chunk)
    if stacked:
        out["forward_call"]["note"] = ("rnn_fwd_%s_stack over %d layers; the recurrence and "
                                       "input projection entries time layer 0's kernels"
                                       % (w.cell, w.layers))
    if not args.no_cpu and lstm and not stacked and not chunked:
        out["cpu_baseline"] = cpu_baseline(w, c, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
