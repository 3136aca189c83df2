#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): the transformer block's O projection
(M = N = K = 4096, bf16 in and out, alpha = 0.5, calibrated on 512 separate
tokens fed as 4 batches of 128). One step is one pass of the whole path
over one batch of synthetic input:
  reset the running max -> 4 x sq_calibrate -> sq_prepare_weight_tiled ->
  sq_quantize_act_tiled -> sq_w8a8_gemm_tiled (int8 GEMM + fused dequant),
the int8 codes kept in 16 x 64 tiles (--layout row: the row-major calls
sq_prepare_weight, sq_quantize_act and sq_w8a8_gemm instead).
Other workloads (--workload) are the remaining shapes of the method's
workloads: prefill, the block's qkv / up / down linears and the MLP
up-projection run the same full step; decode times the per-call path
(sq_quantize_act_tiled + sq_w8a8_gemm_tiled, which streams the weights for
m <= 64) on weights prepared once, as a decode step uses them;
o_proj_per_tensor times the per-tensor variant as its layer runs it
(sq_quantize_tensor_tiled of W and of X, sq_w8a8_gemm_per_tensor_tiled);
decode_weight_only times the weight-only int8 linear (sq_wo_linear_tiled)
on the decode shape. --layout row gives the row-major calls throughout.

Inputs are resident in HBM before the timed region; enough copies of every
buffer a step reads are rotated (at least 512 MiB per cycle, counting the
step's bytes and also the product's alone; 2 to 12 copies) that neither a
step nor a product launch finds its inputs in the 256 MB Infinity Cache
left there by the previous one. The K timed steps are captured into one
HIP graph on the launch stream and replayed once between two HIP events
(no host launch cost between kernels); a second graph of 64 product
launches over the same buffer sets, replayed between events, gives the
product kernel's average duration; an eager pass of the same steps with an
event between stages gives the per-stage breakdown. Prints one JSON line.

The CPU baseline times the CPU oracle (test infrastructure) on a bounded
sample of the same workload on this host.
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

METRIC = "W8A8 SmoothQuant linear TOPS at M=N=K=4096; % of INT8 MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
ROTATE_BYTES = 512 << 20     # bytes read per rotation cycle, at least
GEMM_LAUNCHES = 64           # product launches in the graph that times the product kernel
STAGE_LAUNCHES = 16          # repetitions of a stage in the graph that times it alone
GEMM_SOURCE = os.path.join(ROOT, "w8a8_quantized_linear_sq_amd", "csrc", "sq_gemm.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_o_proj_4096_traffic.md")

# name -> (description, case factory and arguments, mode)
WORKLOADS = {
    "o_proj": ("block O projection, M=N=K=4096, bf16 in/out, alpha=0.5, 512-token calibration in 4 batches",
               ("block_linear", 1), "full"),
    "prefill": ("prefill linear, 2048 tokens x 4096 -> 4096, bf16 in/out, alpha=0.5, calibrated on the same tokens",
                ("prefill",), "full"),
    "decode": ("decode linear, 16 tokens x 4096 -> 11008, bf16 in/out, alpha=0.5, int8 weights prepared once; "
               "per call: activation codes + int8 product + dequant", ("decode",), "per_call"),
    "qkv": ("block QKV projection, 4096 tokens x 4096 -> 12288, bf16, alpha=0.5, 512-token calibration",
            ("block_linear", 0), "full"),
    "up": ("block up projection, 4096 tokens x 4096 -> 11008, bf16, alpha=0.5, 512-token calibration",
           ("block_linear", 2), "full"),
    "down": ("block down projection, 4096 tokens x 11008 -> 4096, bf16, alpha=0.5, 512-token calibration",
             ("block_linear", 3), "full"),
    "mlp_up": ("MLP up-projection, 8192 tokens x 8192 -> 28672, bf16, bias, alpha=0.5 (of the 0.25/0.5/0.75 "
               "sweep), calibrated on the same tokens", ("mlp_up",), "full"),
    "o_proj_per_tensor": ("per-tensor variant on the O projection shape, M=N=K=4096, bf16 in/out: per call the "
                          "weight and the input quantised with one scale each, then the int8 product",
                          ("block_linear", 1), "per_tensor"),
    "decode_weight_only": ("weight-only int8 linear on the decode shape, 16 tokens x 4096 -> 11008, bf16 "
                           "activations and output, per-channel int8 weights prepared once (never calibrated, "
                           "s = 1); per call: the bf16 x int8 product + scale", ("decode",), "weight_only"),
}


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="o_proj")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--layout", choices=("tiled", "row"), default="tiled",
                   help="int8 code layout: 16 x 64 tiles (default) or row-major (the per-tensor workload "
                        "is always row-major)")
    p.add_argument("--counter-pass", action="store_true",
                   help="run only a 256 MiB fp32 copy (known bytes) and the GEMM, 3 times each, for "
                        "rocprofv3 --pmc passes; prints no JSON line")
    return p.parse_args()


def _gemm_traffic(layout: str):
    """HBM bytes per GEMM launch of the O projection from the committed
    rocprofv3 counter summary, or None when the GEMM source changed since
    the counters were taken or they were taken on the other layout."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_l = re.search(r"layout:\s*(\w+)", text)
    if not (m_sha and m_b and m_l) or m_l.group(1) != layout:
        return None
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if sha != m_sha.group(1):
        return None
    return float(m_b.group(1))


def _make_case(inputs, spec):
    return getattr(inputs, spec[0])(*spec[1:])


def cpu_baseline(case, mode: str, budget_s: float):
    """The oracle on this host's cores. Full step: calibration and weight
    preparation in full, then activation quantisation + integer product +
    dequant on as many token rows as fit the time budget, the step time
    extrapolated to all M rows (those stages are linear in the rows).
    Per-call step: activation quantisation + product + dequant of all M rows,
    repeated while the budget lasts."""
    import numpy as np
    import oracle

    o = oracle.get()
    m, n, k = case.m, case.n, case.k
    bias = None if case.bias is None else case.bias.f32
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if mode == "weight_only":
        wq, sw = o.quantize_rows(case.w.f32)
        reps, spent = 0, 0.0
        while reps == 0 or (spent < budget_s and reps < 50):
            tp = time.perf_counter()
            o.wo_linear(case.x.f32, wq, sw, bias)
            spent += time.perf_counter() - tp
            reps += 1
        step_s = spent / reps
        return {"value": round(2.0 * m * n * k / step_s / 1e12, 6), "unit": "TOPS", "cores": threads,
                "kind": "oracle",
                "sample": (f"per-channel int8 weights ({n}x{k}) prepared once, not timed; {reps} calls of all "
                           f"{m} tokens through the weight-only product in binary64 (OpenMP over rows): "
                           f"{step_s:.4f} s per call"),
                "seconds_measured": round(spent, 3)}
    if mode == "per_tensor":
        # both per-tensor quantisations in full (a per-tensor scale needs the
        # whole tensor), then the integer product and dequant on a row sample
        t0 = time.perf_counter()
        wq, sw = o.quantize_tensor(case.w.f32)
        xq, sx = o.quantize_tensor(case.x.f32)
        t1 = time.perf_counter()
        probe = min(m, 16)
        tp = time.perf_counter()
        o.dequant(o.int_gemm(xq[:probe], wq), np.full(probe, sx, np.float32), np.full(n, sw, np.float32), bias)
        per_row = (time.perf_counter() - tp) / probe
        rows = int(min(m, max(16, max(budget_s - (t1 - t0), 1.0) / per_row)))
        tp = time.perf_counter()
        o.dequant(o.int_gemm(xq[:rows], wq), np.full(rows, sx, np.float32), np.full(n, sw, np.float32), bias)
        t_rows = time.perf_counter() - tp
        step_s = (t1 - t0) + t_rows * (m / rows)
        return {"value": round(2.0 * m * n * k / step_s / 1e12, 6), "unit": "TOPS", "cores": threads,
                "kind": "oracle",
                "sample": (f"per-tensor quantisation of W ({n}x{k}) and X ({m}x{k}) in full, then {rows} of {m} "
                           f"token rows through the int8 product (OpenMP over rows) and dequant; step time "
                           f"extrapolated to {m} rows: {step_s:.2f} s"),
                "seconds_measured": round((t1 - t0) + t_rows, 3)}
    t0 = time.perf_counter()
    run = np.zeros(k, np.float32)
    for cb in case.calib:
        o.calibrate(cb.f32, run)
    t1 = time.perf_counter()
    s, wq, sw = o.prepare_weight(case.w.f32, run, 0.5)
    t2 = time.perf_counter()

    def rows_pass(rows):
        tp = time.perf_counter()
        xq, sx = o.quantize_act(case.x.f32[:rows], s)
        acc = o.int_gemm(xq, wq)
        o.dequant(acc, sx, sw, bias)
        return time.perf_counter() - tp

    if mode == "per_call":
        reps, spent = 0, 0.0
        while reps == 0 or (spent < budget_s and reps < 50):
            spent += rows_pass(m)
            reps += 1
        step_s = spent / reps
        sample = (f"weights prepared once ({n}x{k}, not timed, as on the GPU); {reps} per-call passes of "
                  f"all {m} tokens through activation quantisation, the int8 product (OpenMP over rows) "
                  f"and dequant: {step_s:.4f} s per call")
        measured = spent
    else:
        probe = min(m, 16)
        per_row = rows_pass(probe) / probe
        left = max(budget_s - (t2 - t0), 1.0)
        rows = int(min(m, max(16, left / per_row)))
        calib_rows = sum(int(c.f32.shape[0]) for c in case.calib)
        if rows >= m:
            # the whole step fits the budget: whole steps, repeated while the
            # budget lasts (the first one's calibration and preparation are
            # the ones timed above)
            spent, steps = (t2 - t0) + rows_pass(m), 1
            while spent < budget_s and steps < 50:
                tp = time.perf_counter()
                run = np.zeros(k, np.float32)
                for cb in case.calib:
                    o.calibrate(cb.f32, run)
                s, wq, sw = o.prepare_weight(case.w.f32, run, 0.5)
                rows_pass(m)
                spent += time.perf_counter() - tp
                steps += 1
            step_s = spent / steps
            sample = (f"{steps} whole steps: calibration ({calib_rows} tokens), weight preparation ({n}x{k}) "
                      f"and all {m} token rows through activation quantisation, the int8 product (OpenMP "
                      f"over rows) and dequant: {step_s:.3f} s per step")
            measured = spent
        else:
            t_rows = rows_pass(rows)
            step_s = (t1 - t0) + (t2 - t1) + t_rows * (m / rows)
            sample = (f"calibration ({calib_rows} tokens) and weight preparation ({n}x{k}) in full, then "
                      f"{rows} of {m} token rows through activation quantisation, the int8 product (OpenMP "
                      f"over rows) and dequant; step time extrapolated to {m} rows: {step_s:.2f} s")
            measured = (t2 - t0) + t_rows
    return {
        "value": round(2.0 * m * n * k / step_s / 1e12, 6),
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": sample,
        "seconds_measured": round(measured, 3),
    }


def alpha_sweep(torch, B, case, s, stream):
    """The workload's alpha sweep after the timed region (page
    "w8a8_smoothquant.py": recompute_smooth_scale, then quantization_error):
    the weight column max once, the reference linear once (bf16 MFMA, fp32
    out), then per alpha (and for s = 1) the one-pass re-smoothing, the
    quantized forward with fp32 output and the error reduction, all on the
    GPU; the re-smoothing and the reference linear are timed with events."""
    m, n, k = case.m, case.n, case.k
    dev = s["w"].device
    wq = torch.empty((n, k), dtype=torch.int8, device=dev)
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    mw = torch.empty(k, dtype=torch.float32, device=dev)
    y_fp = torch.empty((m, n), dtype=torch.float32, device=dev)
    y_q = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = torch.empty(B.sq_relative_error_workspace_bytes(m * n), dtype=torch.uint8, device=dev)
    res = torch.empty(3, dtype=torch.float64, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    B.sq_weight_col_max(s["w"], mw, stream)
    B.sq_reference_linear(s["x"], s["w"], s["bias"], y_fp, stream)  # warm
    ev[0].record(stream)
    B.sq_reference_linear(s["x"], s["w"], s["bias"], y_fp, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ref_ms = ev[0].elapsed_time(ev[1])
    out = {"reference_linear_us": round(ref_ms * 1e3, 1),
           "reference_linear_tflops_bf16": round(2.0 * m * n * k / (ref_ms * 1e-3) / 1e12, 1),
           "note": "after the timed region; recompute = sq_recompute_smooth_scale (one pass over W)"}
    for alpha in (*case.alphas, None):
        mx = None if alpha is None else s["run"]
        a = 0.5 if alpha is None else alpha
        B.sq_recompute_smooth_scale(s["w"], mx, mw, a, s["smooth"], wq, s["ws"], stream)  # warm
        ev[0].record(stream)
        B.sq_recompute_smooth_scale(s["w"], mx, mw, a, s["smooth"], wq, s["ws"], stream)
        ev[1].record(stream)
        B.sq_quantize_act(s["x"], s["smooth"], xq, s["xs"], stream)
        B.sq_w8a8_gemm(xq, s["xs"], wq, s["ws"], s["bias"], y_q, stream)
        B.sq_relative_error(y_fp, y_q, ws, res, stream)
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[1])
        gbs = (2 * n * k + n * k + 4 * n + 12 * k) / (t * 1e-3) / 1e9
        out["s=1" if alpha is None else f"alpha={alpha}"] = {
            "quantization_error": float(res[2].item()), "recompute_us": round(t * 1e3, 1),
            "recompute_hbm_frac": round(gbs / PEAK_HBM_GBS, 3)}
    return out


def counter_pass(torch, B, s, stream, tiled):
    """A copy of known size (reads and writes 256 MiB: torch.neg over 2^26
    fp32) gives the factor between the HBM counters and real bytes; then the
    product of the benchmark step on prepared operands."""
    src = torch.ones(1 << 26, dtype=torch.float32, device=s["x"].device)
    dst = torch.empty_like(src)
    B.sq_calibrate(s["calib"][0], s["run"], stream)
    m, k = s["x"].shape
    n = s["w"].shape[0]
    if tiled:
        B.sq_prepare_weight_tiled(s["w"], s["run"], 0.5, s["smooth"], s["wq"], s["ws"], stream)
        B.sq_quantize_act_tiled(s["x"], s["smooth"], s["xq"], s["xs"], stream)
    else:
        B.sq_prepare_weight(s["w"], s["run"], 0.5, s["smooth"], s["wq"], s["ws"], stream)
        B.sq_quantize_act(s["x"], s["smooth"], s["xq"], s["xs"], stream)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    for _ in range(3):
        if tiled:
            B.sq_w8a8_gemm_tiled(s["xq"], s["xs"], m, s["wq"], s["ws"], n, k, s["bias"], s["y"], stream)
        else:
            B.sq_w8a8_gemm(s["xq"], s["xs"], s["wq"], s["ws"], s["bias"], s["y"], stream)
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

    import numpy as np
    import torch
    from w8a8_quantized_linear_sq_amd import binding as B
    from w8a8_quantized_linear_sq_amd import inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if libsq.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    desc, spec, mode = WORKLOADS[args.workload]
    case = _make_case(inputs, spec)
    m, n, k = case.m, case.n, case.k
    alpha = 0.5
    # the int8 codes in 16 x 64 tiles unless asked not to
    tiled = args.layout == "tiled"

    def bf16(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x0, w0 = bf16(case.x), bf16(case.w)
    b0 = None if case.bias is None else bf16(case.bias)
    c0 = [bf16(c) for c in case.calib]
    calib_rows = sum(int(c.shape[0]) for c in c0)
    # bytes one step reads and writes (the rotated part)
    if mode == "per_call":
        set_bytes = m * k * 2 + n * k + 4 * n + 4 * k + m * k + m * n * 2
    elif mode == "weight_only":
        set_bytes = m * k * 2 + n * k + 4 * n + m * n * 2
    elif mode == "per_tensor":
        set_bytes = m * k * 2 + n * k * 2 + n * k + m * k + m * n * 2
    else:
        set_bytes = m * k * 2 + n * k * 2 + calib_rows * k * 2 + n * k + m * k + m * n * 2
    # ... and the bytes of one product launch alone (its graph rotates over
    # the same sets): enough sets that neither cycle fits the cache
    gemm_bytes = (m * k + n * k) + m * n * 2 if mode != "weight_only" else n * k + m * k * 2 + m * n * 2
    rotate = max(2, min(12, math.ceil(ROTATE_BYTES / min(set_bytes, gemm_bytes))))
    sets = []
    for _ in range(rotate):
        sets.append(dict(
            x=x0.clone(), w=w0.clone(), calib=[c.clone() for c in c0],
            bias=None if b0 is None else b0.clone(),
            run=torch.zeros(k, dtype=torch.float32, device=dev),
            smooth=torch.empty(k, dtype=torch.float32, device=dev),
            wq=B.tiled_empty(n, k, dev) if tiled else torch.empty((n, k), dtype=torch.int8, device=dev),
            ws=torch.empty(n, dtype=torch.float32, device=dev),
            xq=B.tiled_empty(m, k, dev) if tiled else torch.empty((m, k), dtype=torch.int8, device=dev),
            xs=torch.empty(m, dtype=torch.float32, device=dev),
            y=torch.empty((m, n), dtype=torch.bfloat16, device=dev),
            tsx=torch.empty(1, dtype=torch.float32, device=dev),
            tsw=torch.empty(1, dtype=torch.float32, device=dev)))
    del x0, w0, c0
    # one stream of our own (default priority) for every call, so that the
    # steps can be captured into a graph on it
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    if args.counter_pass:
        counter_pass(torch, B, sets[0], stream, tiled)
        return
    if mode in ("per_call", "weight_only"):
        # weights prepared once per copy, outside the timed region; the bf16
        # weights are then released (weight-only: never calibrated, s = 1)
        prep = B.sq_prepare_weight_tiled if tiled else B.sq_prepare_weight
        for s in sets:
            if mode == "weight_only":
                prep(s["w"], None, alpha, s["smooth"], s["wq"], s["ws"], stream)
                continue
            for cb in s["calib"]:
                B.sq_calibrate(cb, s["run"], stream)
            prep(s["w"], s["run"], alpha, s["smooth"], s["wq"], s["ws"], stream)
        torch.cuda.synchronize()
        for s in sets:
            s["w"] = None
        torch.cuda.empty_cache()
        stage_names = ["quantize_act", "gemm"] if mode == "per_call" else ["wo_linear"]
    elif mode == "per_tensor":
        stage_names = ["quantize_weight", "quantize_act", "gemm"]
    else:
        stage_names = ["reset+calibrate", "prepare_weight", "quantize_act", "gemm"]

    # every call of a step marshalled once per buffer set (binding.prepared):
    # the timed loop then only repeats the C calls
    for s in sets:
        if mode == "per_tensor":
            quant = B.sq_quantize_tensor_tiled if tiled else B.sq_quantize_tensor
            s["call_prep"] = B.prepared(quant, s["w"], s["wq"], s["tsw"], stream)
            s["call_act"] = B.prepared(quant, s["x"], s["xq"], s["tsx"], stream)
            if tiled:
                s["call_gemm"] = B.prepared(B.sq_w8a8_gemm_per_tensor_tiled, s["xq"], s["tsx"], m, s["wq"], s["tsw"],
                                            n, k, s["bias"], s["y"], stream)
            else:
                s["call_gemm"] = B.prepared(B.sq_w8a8_gemm_per_tensor, s["xq"], s["tsx"], s["wq"], s["tsw"],
                                            s["bias"], s["y"], stream)
            continue
        if mode == "weight_only":
            s["call_act"] = None
            if tiled:
                s["call_gemm"] = B.prepared(B.sq_wo_linear_tiled, s["x"], s["wq"], s["ws"], n, s["bias"], s["y"],
                                            stream)
            else:
                s["call_gemm"] = B.prepared(B.sq_wo_linear, s["x"], s["wq"], s["ws"], s["bias"], s["y"], stream)
            continue
        if mode == "full":
            s["calls_calib"] = [B.prepared(B.sq_calibrate, cb, s["run"], stream) for cb in s["calib"]]
        if tiled:
            if mode == "full":
                s["call_prep"] = B.prepared(B.sq_prepare_weight_tiled, s["w"], s["run"], alpha, s["smooth"],
                                            s["wq"], s["ws"], stream)
            s["call_act"] = B.prepared(B.sq_quantize_act_tiled, s["x"], s["smooth"], s["xq"], s["xs"], stream)
            s["call_gemm"] = B.prepared(B.sq_w8a8_gemm_tiled, s["xq"], s["xs"], m, s["wq"], s["ws"], n, k,
                                        s["bias"], s["y"], stream)
            continue
        if mode == "full":
            s["call_prep"] = B.prepared(B.sq_prepare_weight, s["w"], s["run"], alpha, s["smooth"], s["wq"],
                                        s["ws"], stream)
        s["call_act"] = B.prepared(B.sq_quantize_act, s["x"], s["smooth"], s["xq"], s["xs"], stream)
        s["call_gemm"] = B.prepared(B.sq_w8a8_gemm, s["xq"], s["xs"], s["wq"], s["ws"], s["bias"], s["y"], stream)

    def step(i, ev=None):
        s = sets[i % rotate]
        marks = iter(ev) if ev is not None else None

        def mark():
            if marks is not None:
                next(marks).record(stream)

        mark()
        if mode == "full":
            s["run"].zero_()
            for call in s["calls_calib"]:
                call()
            mark()
            s["call_prep"]()
            mark()
        elif mode == "per_tensor":
            s["call_prep"]()
            mark()
        if s["call_act"] is not None:
            s["call_act"]()
            mark()
        s["call_gemm"]()
        mark()

    def new_events(count, per):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(per)] for _ in range(count)]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the K steps are captured into one HIP graph on the launch stream and
    # replayed once as the timed region (no host launch cost between
    # kernels: microsecond-scale steps would otherwise be paced by the host)
    steps_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(steps_graph, stream=stream):
        for i in range(args.steps):
            step(i)
    region = new_events(1, 2)[0]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    region[0].record(stream)
    steps_graph.replay()
    region[1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = region[0].elapsed_time(region[1]) / args.steps

    # the product kernel's average duration: a graph of GEMM_LAUNCHES product
    # launches over the rotated buffer sets, as in the steps, replayed once
    # untimed and once between events on the launch stream
    gemm_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gemm_graph, stream=stream):
        for i in range(GEMM_LAUNCHES):
            sets[i % rotate]["call_gemm"]()
    gemm_graph.replay()
    gev = new_events(1, 2)[0]
    torch.cuda.synchronize()
    gev[0].record(stream)
    gemm_graph.replay()
    gev[1].record(stream)
    torch.cuda.synchronize()
    gemm_ms = gev[0].elapsed_time(gev[1]) / GEMM_LAUNCHES

    # warm: the same launches all on the first buffer set (its operands stay
    # in the 256 MB Infinity Cache when they fit)
    warm_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(warm_graph, stream=stream):
        for i in range(GEMM_LAUNCHES):
            sets[0]["call_gemm"]()
    warm_graph.replay()
    torch.cuda.synchronize()
    gev[0].record(stream)
    warm_graph.replay()
    gev[1].record(stream)
    torch.cuda.synchronize()
    gemm_warm_ms = gev[0].elapsed_time(gev[1]) / GEMM_LAUNCHES

    # stage breakdown: a second pass of K steps with an event between stages
    # (every event adds a few microseconds between kernels, so this pass is
    # not the throughput figure)
    events = new_events(args.steps, len(stage_names) + 1)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, ev=events[i])
    torch.cuda.synchronize()
    stage_ms = {nm: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps
                for j, nm in enumerate(stage_names)}

    # each stage on its own: a graph of STAGE_LAUNCHES repetitions over the
    # rotated buffer sets, replayed untimed and then between events (the
    # per-launch floor between dependent kernels included, no event gaps);
    # these figures give the stages' rooflines
    def stage_calls(s, nm):
        if nm == "reset+calibrate":
            return [s["run"].zero_] + s["calls_calib"]
        if nm in ("prepare_weight", "quantize_weight"):
            return [s["call_prep"]]
        if nm == "quantize_act":
            return [s["call_act"]]
        return [s["call_gemm"]]

    stage_graph_ms = {}
    for nm in stage_names:
        if nm == "gemm":
            stage_graph_ms[nm] = gemm_ms
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(STAGE_LAUNCHES):
                for call in stage_calls(sets[i % rotate], nm):
                    call()
        g.replay()
        torch.cuda.synchronize()
        gev[0].record(stream)
        g.replay()
        gev[1].record(stream)
        torch.cuda.synchronize()
        stage_graph_ms[nm] = gev[0].elapsed_time(gev[1]) / STAGE_LAUNCHES

    ops = 2.0 * m * n * k
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    act_ms = stage_graph_ms.get("quantize_act", 0.0)
    linear_tops = ops / ((act_ms + gemm_ms) * 1e-3) / 1e12

    def hbm(bytes_, ms):
        gbs = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}

    # algorithmic bytes of the HBM-bound stages (a per-tensor scale needs a
    # whole pass over the tensor before its first code: two reads)
    wo_bytes = n * k + m * k * 2 + 2 * m * n + 4 * n
    if mode == "weight_only":
        stage_roof = {"wo_linear": hbm(wo_bytes, stage_graph_ms["wo_linear"])}
    elif mode == "per_tensor":
        stage_roof = {"quantize_act": hbm(2 * m * k * 2 + m * k, act_ms),
                      "quantize_weight": hbm(2 * n * k * 2 + n * k, stage_graph_ms["quantize_weight"])}
    else:
        stage_roof = {"quantize_act": hbm(m * k * 2 + m * k + 4 * m + 4 * k, act_ms)}
    if mode == "full":
        stage_roof["prepare_weight"] = hbm(2 * n * k * 2 + n * k + 4 * n + 8 * k, stage_graph_ms["prepare_weight"])
        stage_roof["reset+calibrate"] = hbm(calib_rows * k * 2 + 8 * k, stage_graph_ms["reset+calibrate"])
    kernel_name = (("int8 GEMM + fused dequant on 16 x 64 tiles (sq_w8a8_gemm_per_tensor_tiled)" if tiled
                    else "int8 GEMM + fused dequant (sq_w8a8_gemm_per_tensor)") if mode == "per_tensor"
                   else "int8 GEMM + fused dequant on 16 x 64 tiles (sq_w8a8_gemm_tiled)" if tiled
                   else "int8 GEMM + fused dequant (sq_w8a8_gemm)")
    if mode == "weight_only":
        # the weight-only product on the decode shape: bound by reading the
        # int8 weights once
        gbs = wo_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": ("weight-only int8 linear on 16 x 64 weight tiles, bf16 MFMA "
                                           "(sq_wo_linear_tiled)" if tiled else
                                           "weight-only int8 linear, bf16 MFMA (sq_wo_linear)"),
                "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    elif m <= 64:
        # the weight-streaming product: bound by reading the int8 weights
        gbs = (n * k + m * k + 2 * m * n + 4 * (m + n)) / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": ("weight-streaming int8 product + fused dequant on 16 x 64 tiles "
                                           "(sq_w8a8_gemm_tiled, m <= 64)" if tiled else
                                           "weight-streaming int8 product + fused dequant (sq_w8a8_gemm, m <= 64)"),
                "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        traffic = _gemm_traffic(args.layout) if args.workload == "o_proj" else None
        roof = {"bound": "mfma", "kernel": kernel_name,
                "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                "traffic": None if traffic is None else round(traffic)}

    config = {"workload": desc, "m": m, "n": n, "k": k, "alpha": alpha, "in_dtype": "bf16",
              "out_dtype": "bf16", "bias": case.bias is not None, "rotated_buffer_sets": rotate}
    if mode == "full":
        config["calib_tokens"] = calib_rows
    config["int8_layout"] = "16x64 tiles" if tiled else "row-major"
    stages = {nm: round(v * 1e3, 2) for nm, v in stage_ms.items()}
    stages["note"] = "second pass of the same K steps with an event between stages"
    stages_graph = {nm: round(v * 1e3, 2) for nm, v in stage_graph_ms.items()}
    stages_graph["note"] = (f"each stage alone: a graph of {STAGE_LAUNCHES} repetitions over the rotated sets "
                            "(the product: its own graph); the stage rooflines use these")
    line = {
        "metric": (METRIC if args.workload == "o_proj" else
                   f"weight-only int8 linear TOPS at M={m} N={n} K={k}" if mode == "weight_only" else
                   f"W8A8 SmoothQuant linear TOPS at M={m} N={n} K={k}"),
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == "weight_only" else "int8",
        "data": "synthetic (seeded; outlier input channels, W ~ N(0, sigma), bf16)",
        "config": config,
        "roofline": roof,
        "gemm_us": round(gemm_ms * 1e3, 2),
        "gemm_launches_timed": GEMM_LAUNCHES,
        "gemm_us_warm": round(gemm_warm_ms * 1e3, 2),
        "stages_us": stages,
        "stages_us_graph": stages_graph,
        "stage_rooflines": stage_roof,
        "linear_tops": round(linear_tops, 2),
        "gemm_tops": round(gemm_tops, 2),
        "wall_s_timed": round(t_wall, 4),
    }
    if mode == "full" and len(case.alphas) > 1:
        line["alpha_sweep"] = alpha_sweep(torch, B, case, sets[0], stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, mode, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
