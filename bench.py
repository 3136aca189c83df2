#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): the transformer block's O projection
(M = N = K = 4096, bf16 in and out, alpha = 0.5, calibrated on 512 separate
tokens fed as 4 batches of 128). One step is one pass of the whole path
over one batch of synthetic input:
  sq_calibrate_batches (the 4 batches in one launch, starting the running
  max) -> sq_prepare_weight_tiled ->
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
import threading
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
    "ste_prefill": ("straight-through backward of the prefill linear, 2048 tokens x 4096 -> 4096, bf16, "
                    "alpha=0.5 calibrated on the same tokens, upstream gradient N(0, 1) bf16 (seed 2010); per "
                    "call: sq_ste_backward (dx, dw, db, ds and the alpha / eta gradient)", ("prefill",), "ste"),
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
    p.add_argument("--no-sclk", action="store_true",
                   help="skip sampling the shader clock and the MFMA-ceiling probe after the timed figures "
                        "(for profiler runs: their launches would outnumber the benchmark's own in a kernel "
                        "trace)")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--layout", choices=("tiled", "row"), default="tiled",
                   help="int8 code layout: 16 x 64 tiles (default) or row-major (the per-tensor workload "
                        "is always row-major)")
    p.add_argument("--counter-pass", action="store_true",
                   help="run only a 256 MiB fp32 copy (known bytes) and the GEMM, 3 times each, for "
                        "rocprofv3 --pmc passes; prints no JSON line")
    p.add_argument("--sweep-k", action="store_true",
                   help="time the tiled int8 product at M = N = 4096 for K = 64 ... 8192 (graphs of 64 "
                        "launches over 8 rotated operand sets, quantised N(0,1) codes, bf16 out): one JSON "
                        "line per K; the intercept is the launch's fixed cost")
    p.add_argument("--hbm-reference", action="store_true",
                   help="time torch's own device copy, fill and column amax at 48 MiB, 192 MiB and 1 GiB "
                        "(graphs of 16 over rotated buffers): the HBM rates plain kernels reach on this box, "
                        "one JSON line")
    p.add_argument("--vendor-reference", action="store_true",
                   help="the vendor library's int8 GEMM (torch._int_mm, int32 out) against this library's "
                        "product (int32 and bf16 out, row-major and tiled) on the O projection's quantised "
                        "codes, 32 launches over 8 rotated sets; one JSON line")
    p.add_argument("--mfma-reference", action="store_true",
                   help="the int8 matrix units' ceiling on this box: the product's own MFMA instructions at "
                        "4096^3 with no memory work (libsq_probe.so), beside the tiled product on the same "
                        "codes, graphs of 64 launches; shader clock per workgroup from s_memtime over "
                        "s_memrealtime; one JSON line")
    return p.parse_args()


def vendor_reference(torch, B, dev):
    """Paired timing, one process: torch._int_mm (the vendor int8 GEMM,
    int32 out) and this library's product on the same codes (the O
    projection's activations and weights quantised by this library), each as
    32 launches over 8 rotated sets; the int32 results compared element for
    element."""
    import numpy as np

    from w8a8_quantized_linear_sq_amd import inputs

    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    case = inputs.o_proj()
    m, n, k = case.m, case.n, case.k
    x0 = torch.from_numpy(case.x.bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(case.w.bits.view(np.int16)).to(dev).view(torch.bfloat16)
    run = torch.zeros(k, dtype=torch.float32, device=dev)
    for cb in case.calib:
        B.sq_calibrate(torch.from_numpy(cb.bits.view(np.int16)).to(dev).view(torch.bfloat16), run, stream)
    sets = []
    for i in range(8):
        s_ = torch.empty(k, device=dev)
        xq, wq = torch.empty((m, k), dtype=torch.int8, device=dev), torch.empty((n, k), dtype=torch.int8, device=dev)
        sx, sw = torch.empty(m, device=dev), torch.empty(n, device=dev)
        B.sq_prepare_weight(w0, run, 0.5, s_, wq, sw, stream)
        B.sq_quantize_act(x0, s_, xq, sx, stream)
        xt, wt = B.tiled_empty(m, k, dev), B.tiled_empty(n, k, dev)
        B.sq_prepare_weight_tiled(w0, run, 0.5, s_, wt, sw, stream)
        B.sq_quantize_act_tiled(x0, s_, xt, sx, stream)
        sets.append(dict(xq=xq, wq=wq, xt=xt, wt=wt, sx=sx, sw=sw,
                         y32=torch.empty((m, n), dtype=torch.int32, device=dev),
                         y16=torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
    del x0, w0
    torch.cuda.synchronize()

    # eager launches (the vendor library refuses stream capture): a pass
    # of 32 untimed, then 32 between events; at ~60 us per launch the host
    # enqueues far ahead of the GPU, so the events time the kernels
    def timed(fn):
        for i in range(32):
            fn(sets[i % 8])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(32):
            fn(sets[i % 8])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / 32

    us = {
        "vendor_int_mm_int32": timed(lambda st: torch._int_mm(st["xq"], st["wq"].t())),
        "sq_w8a8_gemm_int32": timed(lambda st: B.sq_w8a8_gemm(st["xq"], None, st["wq"], None, None, st["y32"],
                                                               stream)),
        "sq_w8a8_gemm_tiled_int32": timed(lambda st: B.sq_w8a8_gemm_tiled(st["xt"], None, m, st["wt"], None, n, k,
                                                                          None, st["y32"], stream)),
        "sq_w8a8_gemm_tiled_bf16": timed(lambda st: B.sq_w8a8_gemm_tiled(st["xt"], st["sx"], m, st["wt"], st["sw"],
                                                                         n, k, None, st["y16"], stream)),
    }
    st = sets[0]
    ref = torch._int_mm(st["xq"], st["wq"].t())
    B.sq_w8a8_gemm_tiled(st["xt"], None, m, st["wt"], None, n, k, None, st["y32"], stream)
    torch.cuda.synchronize()
    ops = 2.0 * m * n * k
    print(json.dumps({"metric": "int8 GEMM at M=N=K=4096 on the O projection's codes (us per launch)",
                      "us": {key: round(v, 2) for key, v in us.items()},
                      "tops": {key: round(ops / (v * 1e-6) / 1e12, 1) for key, v in us.items()},
                      "int32_identical": bool(torch.equal(ref, st["y32"]))}), flush=True)


def hbm_reference(torch, dev):
    """Reference HBM rates of torch's own kernels (not this library's) on
    the box: a device copy (read + write), a fill (write only) and a column
    amax of a bf16 [rows][4096] matrix (read only), each as a graph of 16
    launches over enough rotated buffers that every cycle covers at least
    1 GiB (so no launch finds its data in the 256 MB Infinity Cache),
    replayed once untimed and once between events."""
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    out = {"metric": "reference HBM rates of plain torch kernels (GB/s)", "unit": "GB/s", "sizes_mib": {}}

    def timed(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(16):
                calls[i % len(calls)]()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / 16

    for mib in (48, 192, 1024):
        nbytes = mib << 20
        sets = max(2, -(-(1 << 30) // nbytes))
        src = [torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_() for _ in range(sets)]
        dst = [torch.empty_like(t) for t in src]
        cols = 4096
        red = [torch.empty(cols, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
        torch.cuda.synchronize()
        t_copy = timed([lambda i=i: dst[i].copy_(src[i]) for i in range(sets)])
        t_fill = timed([lambda i=i: dst[i].fill_(1.0) for i in range(sets)])
        t_amax = timed([lambda i=i: torch.amax(src[i].view(-1, cols), dim=0, out=red[i]) for i in range(sets)])
        out["sizes_mib"][str(mib)] = {"copy": round(2 * nbytes / t_copy / 1e9, 1),
                                      "fill": round(nbytes / t_fill / 1e9, 1),
                                      "column_amax": round(nbytes / t_amax / 1e9, 1), "rotated_sets": sets}
        del src, dst, red
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def _probe_lib():
    """libsq_probe.so (the MFMA-ceiling probe), loaded on first use."""
    import ctypes

    from w8a8_quantized_linear_sq_amd import build as hip_build

    if not os.path.exists(hip_build.PROBE_LIB):
        raise RuntimeError(f"{hip_build.PROBE_LIB} is missing: build first (python -m w8a8_quantized_linear_sq_amd.build)")
    P = ctypes.CDLL(hip_build.PROBE_LIB)
    P.sqp_mfma_ceiling.restype = ctypes.c_int
    P.sqp_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.sqp_stream_probe.restype = ctypes.c_int
    P.sqp_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return P


def mfma_ceiling(torch, dev, stream, xq, wq, m, n, k):
    """The matrix units' ceiling for an m x n x k int8 product on this machine,
    measured beside the product: the probe kernel (csrc/sq_probe.hip) issues
    the product's 256 x 256-tile MFMA instructions with no memory work, as a
    graph of 64 launches replayed once untimed and once between events. Its
    operands are bytes of the int8 code buffers xq (m x k) and wq (n x k),
    row-major or in 16 x 64 tiles (the same size when k is a multiple of 64;
    only their values matter). None where the shape does not fit the probe's
    grid (m and n multiples of 256, k of 64) or its 256 x 256 tiles do not
    fill the chip's 256 compute units (the product then runs smaller tiles,
    and the probe's figure would not be its ceiling)."""
    import ctypes

    import numpy as np

    if m % 256 or n % 256 or k % 64 or (m // 256) * (n // 256) < 256:
        return None
    P = _probe_lib()
    tiles = (m // 256) * (n // 256)
    sink = torch.empty(tiles * 512, dtype=torch.int32, device=dev)
    clocks = torch.zeros(5 * tiles, dtype=torch.int64, device=dev)

    def probe():
        rc = P.sqp_mfma_ceiling(xq.data_ptr(), wq.data_ptr(), m, n, k, sink.data_ptr(), clocks.data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"sqp_mfma_ceiling returned {rc}")

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(GEMM_LAUNCHES):
            probe()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / GEMM_LAUNCHES
    cyc = clocks.view(tiles, 5).cpu().numpy()[:, :2].astype(np.float64)
    tops = 2.0 * m * n * k / (us * 1e-6) / 1e12
    del g
    return {"us": round(us, 2), "tops": round(tops, 1), "frac_of_rated_peak": round(tops / PEAK_INT8_TOPS, 4),
            "clock_mhz_median": round(float(np.median(cyc[:, 0] / (cyc[:, 1] / 100.0))), 1),
            "source": "probe kernel (csrc/sq_probe.hip): the product's MFMA instructions with no memory work, "
                      f"graph of {GEMM_LAUNCHES} launches after every timed figure"}


def mfma_reference(torch, B, dev):
    """The ceiling of an int8 product at 4096^3 on this part: the probe
    kernel (csrc/sq_probe.hip) issues the product's MFMA instructions, 16
    per wavefront per 64-byte K step on 256 x 256 tiles, on operands held in
    registers (the codes of the O projection) with no memory work at all.
    Timed as a graph of 64 launches between events, beside the tiled product
    on the same codes: on one operand set (warm, as the probe's own few
    loads are) and over 8 rotated sets (cold, as the default run times it).
    The probe's workgroups report shader cycles and 100 MHz ticks of their
    loop (barrier to barrier), so the clock the chip held and the matrix
    units' busy fraction (32 cycles per instruction per SIMD at the rated
    peak, 2 wavefronts x 16 instructions per step on each SIMD) follow, and
    when the loops started and ended over the grid."""
    import ctypes

    import numpy as np

    from w8a8_quantized_linear_sq_amd import build as hip_build
    from w8a8_quantized_linear_sq_amd import inputs

    P = _probe_lib()
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    case = inputs.o_proj()
    m, n, k = case.m, case.n, case.k
    x0 = torch.from_numpy(case.x.bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(case.w.bits.view(np.int16)).to(dev).view(torch.bfloat16)
    run = torch.zeros(k, dtype=torch.float32, device=dev)
    for cb in case.calib:
        B.sq_calibrate(torch.from_numpy(cb.bits.view(np.int16)).to(dev).view(torch.bfloat16), run, stream)
    s_ = torch.empty(k, device=dev)
    xq, wq = torch.empty((m, k), dtype=torch.int8, device=dev), torch.empty((n, k), dtype=torch.int8, device=dev)
    sx, sw = torch.empty(m, device=dev), torch.empty(n, device=dev)
    B.sq_prepare_weight(w0, run, 0.5, s_, wq, sw, stream)
    B.sq_quantize_act(x0, s_, xq, sx, stream)
    sets = []
    for i in range(8):
        xt, wt = B.tiled_empty(m, k, dev), B.tiled_empty(n, k, dev)
        B.sq_prepare_weight_tiled(w0, run, 0.5, s_, wt, sw, stream)
        B.sq_quantize_act_tiled(x0, s_, xt, sx, stream)
        sets.append((xt, wt, torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
    del x0, w0
    tiles = (m // 256) * (n // 256)
    sink = torch.empty(tiles * 512, dtype=torch.int32, device=dev)
    # two clock buffers, written by alternate launches: the last two launches
    # of a graph give the gap between one launch's end and the next's start
    clocks = [torch.zeros(5 * tiles, dtype=torch.int64, device=dev) for _ in range(2)]
    torch.cuda.synchronize()

    def probe(c, kk=k):
        # kk < k: the same buffers read as kk-byte rows (a prefix of each)
        rc = P.sqp_mfma_ceiling(xq.data_ptr(), wq.data_ptr(), m, n, kk, sink.data_ptr(), c.data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"sqp_mfma_ceiling returned {rc}")

    prods = [B.prepared(B.sq_w8a8_gemm_tiled, xt, sx, m, wt, sw, n, k, None, y, stream) for xt, wt, y in sets]

    def timed(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(GEMM_LAUNCHES):
                calls[r % len(calls)]()
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / GEMM_LAUNCHES

    us_probe = timed([lambda: probe(clocks[0]), lambda: probe(clocks[1])])
    prev, cyc = (c.view(tiles, 5).cpu().numpy() for c in clocks)  # the last two launches
    t0 = cyc[:, 2].min()  # the last launch's first wavefront start

    def rel(v):
        return (v - t0) / 100.0

    entry_us, starts_us, ends_us = rel(cyc[:, 2]), rel(cyc[:, 3]), rel(cyc[:, 4])
    gap_us = (t0 - prev[:, 4].max()) / 100.0
    cyc = cyc[:, :2].astype(np.float64)
    us_probe_k64 = timed([lambda: probe(clocks[0], 64)])
    # the same grid with twice the K (longer launches): codes of 2k bytes a
    # row, the first k bytes of each the O projection's
    xq2 = torch.cat([xq, xq], dim=1)
    wq2 = torch.cat([wq, wq], dim=1)

    def probe_2k():
        rc = P.sqp_mfma_ceiling(xq2.data_ptr(), wq2.data_ptr(), m, n, 2 * k, sink.data_ptr(), clocks[1].data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"sqp_mfma_ceiling returned {rc}")

    us_probe_2k = timed([probe_2k])
    cy2 = clocks[1].view(tiles, 5).cpu().numpy()[:, :2].astype(np.float64)
    probe_2k_line = {"k": 2 * k, "us": round(us_probe_2k, 2),
                     "frac_of_rated_peak": round(4.0 * m * n * k / (us_probe_2k * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
                     "clock_mhz_median": round(float(np.median(cy2[:, 0] / (cy2[:, 1] / 100.0))), 1)}

    # the product's operand stream (tiled codes, direct-to-LDS buffer loads,
    # three steps ahead) alone and with the matrix instructions
    def operand_stream(mfma):
        xt, wt, _ = sets[0]
        rc = P.sqp_stream_probe(xt.data_ptr(), wt.data_ptr(), m, n, k, mfma, sink.data_ptr(), clocks[0].data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"sqp_stream_probe returned {rc}")

    halves = {}
    for name, mfma in (("loads_only", 0), ("loads_and_mfma", 1)):
        us_h = timed([lambda mf=mfma: operand_stream(mf)])
        cy = clocks[0].view(tiles, 5).cpu().numpy()[:, :2].astype(np.float64)
        halves[name] = {"us": round(us_h, 2), "shader_cycles_median": int(np.median(cy[:, 0])),
                        "loop_us_median": round(float(np.median(cy[:, 1])) / 100.0, 2),
                        "clock_mhz_median": round(float(np.median(cy[:, 0] / (cy[:, 1] / 100.0))), 1)}
    us_warm = timed(prods[:1])
    us_cold = timed(prods)
    mhz = cyc[:, 0] / (cyc[:, 1] / 100.0)
    busy = (2 * 16 * (k // 64) * 32) / cyc[:, 0]
    ops = 2.0 * m * n * k

    def tops(us):
        return round(ops / (us * 1e-6) / 1e12, 1)

    print(json.dumps({
        "metric": "int8 MFMA ceiling at M=N=K=4096 (the product's instructions, no memory work) beside the product",
        "probe_us": round(us_probe, 2), "probe_tops": tops(us_probe),
        "probe_frac_of_rated_peak": round(ops / (us_probe * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
        "probe_shader_cycles_median": int(np.median(cyc[:, 0])),
        "probe_clock_mhz_median": round(float(np.median(mhz)), 1),
        "probe_clock_mhz_range": [round(float(mhz.min()), 1), round(float(mhz.max()), 1)],
        "probe_mfma_busy_median": round(float(np.median(busy)), 3),
        "probe_loop_us_median": round(float(np.median(cyc[:, 1])) / 100.0, 2),
        "probe_us_after_first_wave_start": {
            key: [round(float(v.min()), 2), round(float(np.median(v)), 2), round(float(v.max()), 2)]
            for key, v in (("workgroup_start", entry_us), ("loop_start", starts_us), ("end", ends_us))},
        "probe_gap_us_previous_end_to_first_start": round(float(gap_us), 2),
        "probe_us_at_k64": round(us_probe_k64, 2),
        "probe_at_twice_k": probe_2k_line,
        "operand_stream_probe": halves,
        "product_us_warm": round(us_warm, 2), "product_tops_warm": tops(us_warm),
        "product_us_cold": round(us_cold, 2), "product_tops_cold": tops(us_cold),
        "product_over_probe_time_cold": round(us_cold / us_probe, 3),
        "rated_peak_tops": PEAK_INT8_TOPS,
        "note": "graphs of 64 launches; probe clocks from its last launch (min, median, max over workgroups), "
                "the gap from the launch before it; product bf16 out, tiled codes, warm = one operand set, "
                "cold = 8 rotated sets"}), flush=True)


def sweep_k(torch, B, dev):
    """The product's time against K at M = N = 4096: fixed cost and per-step
    cost of the tiled int8 product (each launch the real kernel)."""
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    m = n = 4096
    for k in (64, 128, 256, 512, 1024, 2048, 4096, 8192):
        sets = 8
        ones = torch.ones(k, device=dev)
        # the prepared launches hold raw device pointers only: every set's
        # codes, scales and output stay referenced here until the graph is gone
        bufs, ops = [], []
        for i in range(sets):
            pair = []
            for rows in (m, n):
                x = torch.randn(rows, k, device=dev, generator=gen).to(torch.bfloat16)
                q = B.tiled_empty(rows, k, dev)
                sc = torch.empty(rows, device=dev)
                B.sq_quantize_act_tiled(x, ones, q, sc, stream)
                pair.append((q, sc))
            y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            bufs.append((pair, y))
            ops.append(B.prepared(B.sq_w8a8_gemm_tiled, pair[0][0], pair[0][1], m, pair[1][0], pair[1][1], n, k,
                                  None, y, stream))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(GEMM_LAUNCHES):
                ops[r % sets]()
        g.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / GEMM_LAUNCHES
        print(json.dumps({"sweep": "tiled int8 product, M = N = 4096, bf16 out", "k": k, "us": round(us, 2),
                          "tops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)}), flush=True)
        del g, ops, bufs, ones
        torch.cuda.empty_cache()


def _read_sclk_mhz(path: str):
    """The current shader clock the amdgpu kernel driver reports in pp_dpm_sclk (the line
    marked with '*'), in MHz, or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                    return int(m.group(1)) if m else None
    except OSError:
        return None
    return None


def sample_sclk(load, period_s: float = 0.01):
    """Shader clock while `load()` keeps the GPU busy (it enqueues work and
    waits for it): the amdgpu current-clock file read every period_s from
    a thread of its own; the first fifth of the samples (the clock's ramp)
    is dropped. None where no single such file is readable."""
    import glob
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(files) != 1 or _read_sclk_mhz(files[0]) is None:
        load()
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = _read_sclk_mhz(files[0])
            if v is not None:
                samples.append(v)
            time.sleep(period_s)

    t = threading.Thread(target=sampler, daemon=True)
    t.start()
    try:
        load()
    finally:
        stop.set()
        t.join()
    kept = sorted(samples[len(samples) // 5:])
    if not kept:
        return None
    return {"median": kept[len(kept) // 2], "min": kept[0], "max": kept[-1], "samples": len(kept)}


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


PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def cpu_baseline_ste(case, dy, budget_s: float):
    """The oracle's straight-through backward (binary64) on the first tokens
    of the batch: its own calibration and weight preparation first (not
    timed), then the backward of as many tokens as fit the budget."""
    import oracle

    o = oracle.get()
    m, n, k = case.m, case.n, case.k
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    x, w = case.x.f32, case.w.f32
    mx = o.calibrate(x)
    mw = o.weight_col_max(w)
    s, wq, sw = o.prepare_weight(w, mx, 0.5)

    def run(rows):
        xq, sx = o.quantize_act(x[:rows], s)
        tp = time.perf_counter()
        o.ste_backward(dy.f32[:rows], x[:rows], w, s, xq, sx, wq, sw, mx, mw, 0.5)
        return time.perf_counter() - tp

    probe = 4
    per_row = run(probe) / probe
    rows = int(min(m, max(probe, budget_s / per_row)))
    t = run(rows)
    return {"value": round(4.0 * rows * n * k / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"the oracle's straight-through backward (binary64) on the first {rows} of {m} tokens "
                       f"against the whole {n}x{k} weight (the two products' 4*{rows}*N*K flops, the column, "
                       f"bias and alpha terms included), after its own calibration and weight preparation "
                       f"(not timed): {t:.2f} s"),
            "seconds_measured": round(t, 3)}


def ste_bench(args, torch, np, B, inputs, case, desc, dev):
    """One step = one straight-through backward call (sq_ste_backward) on a
    quantised forward's state prepared beforehand (calibration on the same
    tokens, weight preparation, activation codes: not timed)."""
    m, n, k = case.m, case.n, case.k
    alpha = 0.5
    dy_t = inputs.upstream_grad(m, n, seed=2010)

    def bf16(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x0, w0, dy0 = bf16(case.x), bf16(case.w), bf16(dy_t)
    ws_bytes = B.sq_ste_backward_workspace_bytes(m, n, k)
    set_bytes = m * n * 2 + (m + n) * k * (2 + 1 + 4) + ws_bytes
    rotate = max(2, min(12, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = []
    for _ in range(rotate):
        sets.append(dict(
            dy=dy0.clone(), x=x0.clone(), w=w0.clone(),
            run=torch.empty(k, dtype=torch.float32, device=dev), mw=torch.empty(k, dtype=torch.float32, device=dev),
            smooth=torch.empty(k, dtype=torch.float32, device=dev),
            wq=torch.empty((n, k), dtype=torch.int8, device=dev), ws=torch.empty(n, dtype=torch.float32, device=dev),
            xq=torch.empty((m, k), dtype=torch.int8, device=dev), xs=torch.empty(m, dtype=torch.float32, device=dev),
            dx=torch.empty((m, k), dtype=torch.float32, device=dev),
            dw=torch.empty((n, k), dtype=torch.float32, device=dev),
            db=torch.empty(n, dtype=torch.float32, device=dev), ds=torch.empty(k, dtype=torch.float32, device=dev),
            da=torch.empty(2, dtype=torch.float64, device=dev),
            wsp=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)))
    del x0, w0, dy0
    # the copies above ran on the default stream; the calls below run on a
    # stream of our own, which must not start before them
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    for s in sets:
        B.sq_calibrate_first(s["x"], s["run"], stream)
        B.sq_weight_col_max(s["w"], s["mw"], stream)
        B.sq_prepare_weight(s["w"], s["run"], alpha, s["smooth"], s["wq"], s["ws"], stream)
        B.sq_quantize_act(s["x"], s["smooth"], s["xq"], s["xs"], stream)
        s["call"] = B.prepared(B.sq_ste_backward, s["dy"], s["x"], s["w"], s["smooth"], s["xq"], s["xs"], s["wq"],
                               s["ws"], s["run"], s["mw"], alpha, s["dx"], s["dw"], s["db"], s["ds"], s["da"],
                               s["wsp"], stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        sets[i % rotate]["call"]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(args.steps):
            sets[i % rotate]["call"]()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev[0].record(stream)
    g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = ev[0].elapsed_time(ev[1]) / args.steps
    # the auxiliary loss and its gradient at Y_q (after the timed region):
    # the two norms need a whole pass over Y_fp and Y_q before the first
    # gradient element, so 2 reads of each and one write of M x N fp32
    aux_ws = B.sq_aux_loss_grad_workspace_bytes(m * n)
    for i, s in enumerate(sets):
        gen = torch.Generator(device=dev)
        gen.manual_seed(2020 + i)
        s["y_fp"] = torch.randn(m, n, device=dev, generator=gen)
        s["y_q"] = s["y_fp"] + 0.01 * torch.randn(m, n, device=dev, generator=gen)
        s["dy_q"] = torch.empty(m, n, dtype=torch.float32, device=dev)
        s["loss"] = torch.empty(1, dtype=torch.float64, device=dev)
        s["aux_ws"] = torch.empty(max(aux_ws, 16), dtype=torch.uint8, device=dev)
        s["aux"] = B.prepared(B.sq_aux_loss_grad, s["y_fp"], s["y_q"], s["dy_q"], s["loss"], s["aux_ws"], stream)
    torch.cuda.synchronize()
    ag = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ag, stream=stream):
        for i in range(STAGE_LAUNCHES):
            sets[i % rotate]["aux"]()
    ag.replay()
    torch.cuda.synchronize()
    ev[0].record(stream)
    ag.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    aux_ms = ev[0].elapsed_time(ev[1]) / STAGE_LAUNCHES
    aux_bytes = 5 * m * n * 4
    aux_gbs = aux_bytes / (aux_ms * 1e-3) / 1e9
    flops = 4.0 * m * n * k            # the backward's two products, 2*M*N*K each
    mfma_flops = 12.0 * m * n * k      # as run: each fp32 factor split into three exact bf16 planes
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = mfma_flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": f"straight-through backward TFLOP/s at M={m} N={n} K={k} (two products of 2*M*N*K)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; outlier input channels, W ~ N(0, sigma), upstream gradient N(0, 1), bf16)",
        "config": {"workload": desc, "m": m, "n": n, "k": k, "alpha": alpha, "in_dtype": "bf16",
                   "grad_dtype": "fp32", "rotated_buffer_sets": rotate, "int8_layout": "row-major"},
        "roofline": {"bound": "mfma",
                     "kernel": ("the straight-through backward call: its two products as three exact bf16 "
                                "planes each on bf16 MFMA (gemm_kernel<bf16, .., periodic B>), with the packing "
                                "and column passes; achieved counts the products' 12*M*N*K bf16 MFMA flops over "
                                "the whole call"),
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "call_us": round(ms_per_step * 1e3, 2),
        "aux_loss_grad": {"us": round(aux_ms * 1e3, 2), "bound": "hbm", "achieved": round(aux_gbs, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(aux_gbs / PEAK_HBM_GBS, 4),
                          "note": (f"sq_aux_loss_grad on {m}x{n} fp32 Y_fp / Y_q: two passes over both (the "
                                   f"norms first) and the gradient written, {aux_bytes} bytes per call; "
                                   f"{STAGE_LAUNCHES} calls in one graph over the rotated sets, after the "
                                   "timed region")},
        "wall_s_timed": round(t_wall, 4),
        "value_is": "one backward call per unit time, counting the two products' 4*M*N*K flops",
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_ste(case, dy_t, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


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
    if args.sweep_k:
        sweep_k(torch, B, dev)
        return
    if args.hbm_reference:
        hbm_reference(torch, dev)
        return
    if args.vendor_reference:
        vendor_reference(torch, B, dev)
        return
    if args.mfma_reference:
        mfma_reference(torch, B, dev)
        return

    desc, spec, mode = WORKLOADS[args.workload]
    case = _make_case(inputs, spec)
    if mode == "ste":
        ste_bench(args, torch, np, B, inputs, case, desc, dev)
        return
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
    # the copies and fills above ran on the default stream; every call below
    # runs on a stream of our own (default priority, so that the steps can be
    # captured into a graph on it), which must not start before them
    torch.cuda.synchronize()
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
        stage_names = ["calibrate", "prepare_weight", "quantize_act", "gemm"]

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
            s["calls_calib"] = [B.prepared(B.sq_calibrate_batches, s["calib"], s["run"], True, stream)]
            # the same calibration a batch at a time (timed as a stage of
            # its own, beside the step)
            s["calls_calib_each"] = [B.prepared(B.sq_calibrate_first if i == 0 else B.sq_calibrate, cb, s["run"],
                                                stream) for i, cb in enumerate(s["calib"])]
        if tiled:
            if mode == "full":
                s["call_prep"] = B.prepared(B.sq_prepare_weight_tiled, s["w"], s["run"], alpha, s["smooth"],
                                            s["wq"], s["ws"], stream)
            s["call_act"] = B.prepared(B.sq_quantize_act_tiled, s["x"], s["smooth"], s["xq"], s["xs"], stream)
            s["call_gemm"] = B.prepared(B.sq_w8a8_gemm_tiled, s["xq"], s["xs"], m, s["wq"], s["ws"], n, k,
                                        s["bias"], s["y"], stream)
            if mode == "per_call" and m <= 64:
                # the same forward as one kernel (sq_w8a8_linear_tiled_fused:
                # the weight stream quantises the activations itself)
                s["fws"] = B.linear_tiled_workspace(m, k, dev, fused=True)
                s["call_fused"] = B.prepared(B.sq_w8a8_linear_tiled_fused, s["x"], s["smooth"], s["wq"], s["ws"],
                                             n, s["bias"], s["y"], s["fws"], stream)
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
            # every calibration batch in one call, which starts the running
            # max (no zero fill)
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

    # the per-call linear (the second throughput figure): activation codes + the
    # product, as a forward runs them on prepared weights, GEMM_LAUNCHES
    # calls in one graph over the rotated sets, replayed between events
    per_call_ms = None
    if mode in ("full", "per_call"):
        pc_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pc_graph, stream=stream):
            for i in range(GEMM_LAUNCHES):
                sets[i % rotate]["call_act"]()
                sets[i % rotate]["call_gemm"]()
        pc_graph.replay()
        torch.cuda.synchronize()
        gev[0].record(stream)
        pc_graph.replay()
        gev[1].record(stream)
        torch.cuda.synchronize()
        per_call_ms = gev[0].elapsed_time(gev[1]) / GEMM_LAUNCHES
    fused_ms = None
    if "call_fused" in sets[0]:
        f_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(f_graph, stream=stream):
            for i in range(GEMM_LAUNCHES):
                sets[i % rotate]["call_fused"]()
        f_graph.replay()
        torch.cuda.synchronize()
        gev[0].record(stream)
        f_graph.replay()
        gev[1].record(stream)
        torch.cuda.synchronize()
        fused_ms = gev[0].elapsed_time(gev[1]) / GEMM_LAUNCHES

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
        if nm == "calibrate":
            return s["calls_calib"]
        if nm == "calibrate_each_batch":
            return s["calls_calib_each"]
        if nm in ("prepare_weight", "quantize_weight"):
            return [s["call_prep"]]
        if nm == "quantize_act":
            return [s["call_act"]]
        return [s["call_gemm"]]

    stage_graph_ms = {}
    for nm in stage_names + (["calibrate_each_batch"] if mode == "full" else []):
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

    # the shader clock under the product: the rotated-set product graph
    # replayed back to back for about half a second while the amdgpu
    # current-clock reading is sampled (after every timed figure: the
    # sustained load heats the chip and lowers the clock of what follows)
    replays = max(1, int(0.5 / max(gemm_ms * 1e-3 * GEMM_LAUNCHES, 1e-6)))

    def product_load():
        for _ in range(replays):
            gemm_graph.replay()
        torch.cuda.synchronize()

    sclk = None if args.no_sclk else sample_sclk(product_load)
    if sclk is not None:
        sclk["source"] = (f"pp_dpm_sclk read every 10 ms over {replays} replays of the {GEMM_LAUNCHES}-launch "
                          "product graph (rotated sets)")
        if m > 64 and mode != "weight_only":
            # the product's fraction of the peak scaled to that clock (the
            # rated peak assumes 2.4 GHz)
            at_clock = PEAK_INT8_TOPS * sclk["median"] / 2400.0
            sclk["gemm_frac_of_peak_at_median_clock"] = round(2.0 * m * n * k / (gemm_ms * 1e-3) / 1e12 / at_clock,
                                                              4)

    ops = 2.0 * m * n * k
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    act_ms = stage_graph_ms.get("quantize_act", 0.0)

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
        stage_roof["calibrate"] = hbm(calib_rows * k * 2 + 8 * k, stage_graph_ms["calibrate"])
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
        if sclk is not None and "gemm_frac_of_peak_at_median_clock" in sclk:
            # the same against the peak at the clock the chip held under the
            # product (the rated peak assumes 2.4 GHz)
            roof["sclk_mhz"] = sclk["median"]
            roof["frac_at_sclk"] = sclk["gemm_frac_of_peak_at_median_clock"]
        from w8a8_quantized_linear_sq_amd import build as hip_build
        if not args.no_sclk and not os.path.exists(hip_build.PROBE_LIB):
            # a measurement aid, not the product: its absence is reported
            roof["mfma_ceiling"] = {"skipped": f"{hip_build.PROBE_LIB} not built"}
        elif not args.no_sclk:
            # what the matrix units deliver here with no memory work at all
            ceil = mfma_ceiling(torch, dev, stream, sets[0]["xq"], sets[0]["wq"], m, n, k)
            if ceil is not None:
                roof["mfma_ceiling"] = ceil
                roof["frac_of_ceiling"] = round(ceil["us"] / (gemm_ms * 1e3), 4)

    config = {"workload": desc, "m": m, "n": n, "k": k, "alpha": alpha, "in_dtype": "bf16",
              "out_dtype": "bf16", "bias": case.bias is not None, "rotated_buffer_sets": rotate}
    if mode == "full":
        config["calib_tokens"] = calib_rows
    config["int8_layout"] = "16x64 tiles" if tiled else "row-major"
    stages = {nm: round(v * 1e3, 2) for nm, v in stage_ms.items()}
    stages["note"] = "second pass of the same K steps with an event between stages"
    stages_graph = {nm: round(v * 1e3, 2) for nm, v in stage_graph_ms.items()}
    stages_graph["note"] = (f"each stage alone: a graph of {STAGE_LAUNCHES} repetitions over the rotated sets "
                            "(the product: its own graph); the stage rooflines use these"
                            + ("; calibrate is the step's one sq_calibrate_batches call, calibrate_each_batch the "
                               "same batches a call each (not in the step)" if mode == "full" else ""))
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
        "sclk_mhz_under_gemm": sclk,
        "stages_us": stages,
        "stages_us_graph": stages_graph,
        "stage_rooflines": stage_roof,
        "gemm_tops": round(gemm_tops, 2),
        "wall_s_timed": round(t_wall, 4),
    }
    if per_call_ms is not None:
        line["per_call_linear_us"] = round(per_call_ms * 1e3, 2)
        line["per_call_linear_tops"] = round(ops / (per_call_ms * 1e-3) / 1e12, 2)
        line["per_call_note"] = ("activation codes + int8 product + dequant on prepared weights "
                                 f"({'sq_quantize_act_tiled + sq_w8a8_gemm_tiled' if tiled else 'sq_quantize_act + sq_w8a8_gemm'}), "
                                 f"{GEMM_LAUNCHES} calls in one graph over the rotated sets")
    if fused_ms is not None:
        line["per_call_fused_us"] = round(fused_ms * 1e3, 2)
        line["per_call_fused_tops"] = round(ops / (fused_ms * 1e-3) / 1e12, 2)
        line["per_call_fused_note"] = ("the same forward as one kernel, sq_w8a8_linear_tiled_fused (the weight "
                                       f"stream quantises the activations itself), {GEMM_LAUNCHES} calls in one "
                                       "graph over the rotated sets")
        line["per_call_fused_fallbacks"] = sum(B.linear_tiled_fallbacks(s["fws"]) for s in sets)
    line["value_is"] = ("the whole step (calibration, weight preparation, activation codes, product) per "
                        "unit time" if mode == "full" else "one call per unit time")
    if mode == "full" and len(case.alphas) > 1:
        line["alpha_sweep"] = alpha_sweep(torch, B, case, sets[0], stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, mode, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
