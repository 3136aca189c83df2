#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole path over one batch of synthetic input, on
the transformer block's O projection (M = N = K = 4096, bf16 in and out,
alpha = 0.5, calibrated on 512 separate tokens fed as 4 batches of 128):
  reset the running max -> 4 x sq_calibrate -> sq_prepare_weight ->
  sq_quantize_act -> sq_w8a8_gemm (int8 GEMM + fused dequant).
Inputs are resident in HBM before the timed region; 4 copies of every buffer
are rotated so that each step's data is not left in the 256 MB Infinity
Cache by the previous step. HIP events on the launch stream bracket the
timed region and every GEMM launch in it; a second pass of the same steps
with an event between stages gives the per-stage breakdown. Prints one JSON
line.

The CPU baseline times the CPU oracle (test infrastructure) on a bounded
sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 SmoothQuant linear TOPS at M=N=K=4096; % of INT8 MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
ROTATE = 4
GEMM_SOURCE = os.path.join(ROOT, "w8a8_quantized_linear_sq_amd", "csrc", "sq_gemm.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_o_proj_4096_traffic.md")


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--counter-pass", action="store_true",
                   help="run only a 256 MiB fp32 copy (known bytes) and the GEMM, 3 times each, for "
                        "rocprofv3 --pmc passes; prints no JSON line")
    return p.parse_args()


def _gemm_traffic(gemm_launch_count_bytes=None):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when the GEMM source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if sha != m_sha.group(1):
        return None
    return float(m_b.group(1))


def cpu_baseline(case, budget_s: float):
    """The oracle on this host's cores: calibration and weight preparation in
    full, then activation quantisation + integer GEMM + dequant on as many
    token rows as fit the time budget; the step time is extrapolated to all
    M rows (those stages are linear in the rows)."""
    import numpy as np
    import oracle

    o = oracle.get()
    m, n, k = case.m, case.n, case.k
    t0 = time.perf_counter()
    run = np.zeros(k, np.float32)
    for cb in case.calib:
        o.calibrate(cb.f32, run)
    t1 = time.perf_counter()
    s, wq, sw = o.prepare_weight(case.w.f32, run, 0.5)
    t2 = time.perf_counter()
    # probe 64 rows to size the sample
    rows = 64
    tp = time.perf_counter()
    xq, sx = o.quantize_act(case.x.f32[:rows], s)
    acc = o.int_gemm(xq, wq)
    o.dequant(acc, sx, sw, None)
    per_row = (time.perf_counter() - tp) / rows
    left = max(budget_s - (t2 - t0), 1.0)
    rows = int(min(m, max(64, left / per_row)))
    tp = time.perf_counter()
    xq, sx = o.quantize_act(case.x.f32[:rows], s)
    acc = o.int_gemm(xq, wq)
    o.dequant(acc, sx, sw, None)
    t_rows = time.perf_counter() - tp
    step_s = (t1 - t0) + (t2 - t1) + t_rows * (m / rows)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": round(2.0 * m * n * k / step_s / 1e12, 6),
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"calibration (512 tokens) and weight preparation ({n}x{k}) in full, then "
                   f"{rows} of {m} token rows through activation quantisation, the int8 product "
                   f"(OpenMP over rows) and dequant; step time extrapolated to {m} rows: "
                   f"{step_s:.2f} s"),
        "seconds_measured": round((t2 - t0) + t_rows, 3),
    }


def counter_pass(torch, B, s, dev, stream):
    """A copy of known size (reads and writes 256 MiB: torch.neg over 2^26
    fp32) gives the factor between the HBM counters and real bytes; then the
    GEMM of the benchmark step on prepared operands."""
    src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    B.sq_calibrate(s["calib"][0], s["run"], stream)
    B.sq_prepare_weight(s["w"], s["run"], 0.5, s["smooth"], s["wq"], s["ws"], stream)
    B.sq_quantize_act(s["x"], s["smooth"], s["xq"], s["xs"], stream)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    for _ in range(3):
        B.sq_w8a8_gemm(s["xq"], s["xs"], s["wq"], s["ws"], None, s["y"], stream)
    torch.cuda.synchronize()
    print("counter pass done", flush=True)


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the SmoothQuant W8A8 path "
              "is built and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py does not run under a multi-rank launcher", file=sys.stderr)
        sys.exit(2)

    import torch
    from w8a8_quantized_linear_sq_amd import binding as B
    from w8a8_quantized_linear_sq_amd import inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if libsq.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    case = inputs.o_proj()
    m, n, k = case.m, case.n, case.k
    alpha = 0.5

    def bf16(t):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x0, w0 = bf16(case.x), bf16(case.w)
    c0 = [bf16(c) for c in case.calib]
    sets = []
    for r in range(ROTATE):
        sets.append(dict(
            x=x0.clone(), w=w0.clone(), calib=[c.clone() for c in c0],
            run=torch.zeros(k, dtype=torch.float32, device=dev),
            smooth=torch.empty(k, dtype=torch.float32, device=dev),
            wq=torch.empty((n, k), dtype=torch.int8, device=dev),
            ws=torch.empty(n, dtype=torch.float32, device=dev),
            xq=torch.empty((m, k), dtype=torch.int8, device=dev),
            xs=torch.empty(m, dtype=torch.float32, device=dev),
            y=torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
    del x0, w0, c0
    stream = torch.cuda.current_stream(dev)
    if args.counter_pass:
        counter_pass(torch, B, sets[0], dev, stream)
        return
    n_stage = 5  # reset+calibrate, prepare, act quant, gemm

    def step(i, ev=None, gemm_ev=None):
        s = sets[i % ROTATE]
        if ev is not None:
            ev[0].record(stream)
        s["run"].zero_()
        for cb in s["calib"]:
            B.sq_calibrate(cb, s["run"], stream)
        if ev is not None:
            ev[1].record(stream)
        B.sq_prepare_weight(s["w"], s["run"], alpha, s["smooth"], s["wq"], s["ws"], stream)
        if ev is not None:
            ev[2].record(stream)
        B.sq_quantize_act(s["x"], s["smooth"], s["xq"], s["xs"], stream)
        if ev is not None:
            ev[3].record(stream)
        if gemm_ev is not None:
            gemm_ev[0].record(stream)
        B.sq_w8a8_gemm(s["xq"], s["xs"], s["wq"], s["ws"], None, s["y"], stream)
        if ev is not None:
            ev[4].record(stream)
        if gemm_ev is not None:
            gemm_ev[1].record(stream)

    def new_events(count, per):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(per)] for _ in range(count)]

    for i in range(args.warmup):
        step(i)
    # timed region: K steps; HIP events on the launch stream bracket the
    # region and every GEMM launch (the GEMM's live average duration)
    region = new_events(1, 2)[0]
    gemm_events = new_events(args.steps, 2)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        step(i, gemm_ev=gemm_events[i])
    region[1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = region[0].elapsed_time(region[1]) / args.steps
    gemm_ms = sum(e[0].elapsed_time(e[1]) for e in gemm_events) / args.steps

    # stage breakdown: a second pass of K steps with an event between stages
    # (every event adds a few microseconds between kernels, so this pass is
    # not the throughput figure)
    events = new_events(args.steps, n_stage)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, ev=events[i])
    torch.cuda.synchronize()
    stage_ms = [sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps for j in range(n_stage - 1)]
    calib_ms, prep_ms, act_ms, gemm_stage_ms = stage_ms
    ops = 2.0 * m * n * k
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    linear_tops = ops / ((act_ms + gemm_ms) * 1e-3) / 1e12
    # algorithmic bytes of the HBM-bound stages
    act_bytes = m * k * 2 + m * k + 4 * m + 4 * k
    prep_bytes = 2 * n * k * 2 + n * k + 4 * n + 8 * k
    calib_bytes = 512 * k * 2 + 8 * k
    traffic = _gemm_traffic()

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; 1% outlier input channels x50, W ~ N(0, 0.02), bf16)",
        "config": {"workload": "block O projection, M=N=K=4096, bf16 in/out, alpha=0.5, "
                               "512-token calibration in 4 batches",
                   "m": m, "n": n, "k": k, "alpha": alpha, "in_dtype": "bf16", "out_dtype": "bf16",
                   "calib_tokens": 512, "rotated_buffer_sets": ROTATE},
        "roofline": {"bound": "mfma", "kernel": "int8 GEMM + fused dequant (sq_w8a8_gemm)",
                     "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "gemm_us": round(gemm_ms * 1e3, 2),
        "stages_us": {"reset+calibrate": round(calib_ms * 1e3, 2), "prepare_weight": round(prep_ms * 1e3, 2),
                      "quantize_act": round(act_ms * 1e3, 2), "gemm": round(gemm_stage_ms * 1e3, 2),
                      "note": "second pass of the same K steps with an event between stages"},
        "stage_rooflines": {
            "quantize_act": {"bound": "hbm", "achieved": round(act_bytes / (act_ms * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(act_bytes / (act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "prepare_weight": {"bound": "hbm", "achieved": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(prep_bytes / (prep_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "reset+calibrate": {"bound": "hbm", "achieved": round(calib_bytes / (calib_ms * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s"},
        },
        "linear_tops": round(linear_tops, 2),
        "gemm_tops": round(gemm_tops, 2),
        "wall_s_timed": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
