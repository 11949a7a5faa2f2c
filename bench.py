#!/usr/bin/env python3
"""Throughput of the fused stencil kernels on one MI355X.

One step = one pass of every operation of the library over its full-size
synthetic workload, on inputs already resident in HBM:
  conv        x fp32 [128,8,256,256] -> conv 8->64 k3 + tanh + *2 + bias + maxpool 4
              -> [128,64,63,63]        (74.91 GFLOP: the 252x252 conv outputs the pool reads)
  maxpool     x fp32 [32,64,512,512] -> k4 s1 p1 d1 -> [32,64,511,511]
              (4.2866 GB: every input read once + every output written once)
  convT       x fp32 [128,64,64,64] -> convT 64->128 k4 s2 p1 op1 + softmax + bias + *2
              + sigmoid -> [128,128,129,129]   (136.37 GFLOP over the valid taps)
  conv_bf16   the conv workload with bf16 x, w and output (74.91 GFLOP)
  maxpool_s2  the max-pool input, k3 s2 p1 (downsampling) -> [32,64,256,256]
              (2.147 GB read + 0.537 GB written)
  maxpool_d2  the max-pool input, k3 s1 p2 d2 (dilated) -> [32,64,512,512]
              (2.147 GB read + 2.147 GB written)
  convT_bf16  the convT workload with bf16 x, w and output (fp32 accumulation); bound by
              its HBM bytes (0.613 GB) more than by its 136.37 GFLOP at the bf16 peak
  conv_2stage the conv workload unfused: ps_conv2d stores the full 254x254 conv output
              (2.11 GB), then the epilogue + pool kernel reads it back (the pages' baseline)
  convT_2stage the convT workload unfused: ps_convT2d stores the 1.09 GB output, then
              the softmax post-process runs in place on it
  conv_general x fp32 [32,64,128,128] -> conv 64->128 k3 p1 + tanh + *2 + bias
              + maxpool k3 s2 p1 (overlapping windows) -> [32,128,64,64]
              (77.31 GFLOP: every 128x128 conv output is read by some window)
  tiny_conv   x fp32 [2,8,32,32] -> conv 8->16 k3 + tanh + *2 + bias + maxpool 4
              -> [2,16,7,7] (3.61 MFLOP: a launch-latency-bound call, reported in us)

`value` is the fused conv+maxpool throughput (GFLOP/s, fp32) -- the first
figure of the headline metric; the max-pool's GB/s (the second figure) and the
other two operations are reported in `ops` of the same line, each with its
roofline fraction.  Per-kernel times come from HIP events recorded on the
stream the kernels run on (torch's current stream), averaged over the timed
steps.  Each operation also carries `cpu_baseline`: the CPU oracle (plain C,
double precision, OpenMP) timed on the host cores on a bounded slice of the
same workload, with the host's CPU model and thread counts.  The line also
records the GPU clocks rocm-smi reports while the fused conv runs and the
bandwidth of a plain device copy (a practical HBM ceiling next to 8 TB/s).
Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32 = 157.3e12      # MI355X dense fp32 (vector or matrix), FLOP/s
PEAK_BF16 = 2.5e15        # MI355X dense bf16 matrix, FLOP/s
PEAK_HBM = 8.0e12         # MI355X HBM3E, B/s

CONV_FLOP = 2 * 72 * 128 * 64 * 252 * 252
CONV_FLOP_PAGE = 2 * 72 * 128 * 64 * 254 * 254     # the page's count over all 254x254 outputs
POOL_BYTES = 32 * 64 * 512 * 512 * 4 + 32 * 64 * 511 * 511 * 4
CONV_GENERAL_FLOP = 2 * 64 * 9 * 32 * 128 * 128 * 128
POOL_S2_BYTES = 32 * 64 * 512 * 512 * 4 + 32 * 64 * 256 * 256 * 4
POOL_D2_BYTES = 2 * 32 * 64 * 512 * 512 * 4
CONV_INTER_BYTES = 128 * 64 * 254 * 254 * 4        # the stored conv output of the unfused pipeline
CONVT_INTER_BYTES = 128 * 128 * 129 * 129 * 4      # the stored convT output
CONVT_FLOP = 2 * 128 * 64 * 128 * 255 * 255
CONVT_BYTES = 128 * 64 * 64 * 64 * 4 + 128 * 128 * 129 * 129 * 4 + 64 * 128 * 16 * 4
CONVT_BF16_BYTES = 128 * 64 * 64 * 64 * 2 + 128 * 128 * 129 * 129 * 2 + 64 * 128 * 16 * 2
TINY_FLOP = 2 * 72 * 2 * 16 * 28 * 28              # the 28x28 conv outputs the pool reads

# HBM bytes per launch, from two rocprofv3 --pmc passes over this script (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a
# device copy of known size (`bench.py --copy-calibration`): FETCH_SIZE x2.0, WRITE_SIZE
# x1.0.  `src` is the hash of the kernel's sources when the counters were taken; a
# kernel edited since then reports traffic null.  See profiles/traffic_*.md.
TRAFFIC = {
    "conv": {"src": "024f76aa6b42ecd9", "fetch_bytes": 266662568, "write_bytes": 130646656},
    "conv_bf16": {"src": "024f76aa6b42ecd9", "fetch_bytes": 136674025, "write_bytes": 80061744},
    "maxpool": {"src": "7fe7bbddd12793d9", "fetch_bytes": 2160264806, "write_bytes": 2140710736},
    "maxpool_s2": {"src": "7fe7bbddd12793d9", "fetch_bytes": 2176852435, "write_bytes": 536870912},
    "maxpool_d2": {"src": "7fe7bbddd12793d9", "fetch_bytes": 2266660825, "write_bytes": 2147483648},
    "convT": {"src": "6bcf64774038c99d", "fetch_bytes": 142739559, "write_bytes": 1257164144},
    "convT_bf16": {"src": "795616b272b40138", "fetch_bytes": 78763430, "write_bytes": 773598880},
    "conv_general": {"src": "456ad05d0ed2d488", "fetch_bytes": 137129498, "write_bytes": 69352656},
    "conv_2stage#0": {"src": "8cfb246101a56548", "fetch_bytes": 276823971, "write_bytes": 2116772048},
    "conv_2stage#1": {"src": "8cfb246101a56548", "fetch_bytes": 2112061421, "write_bytes": 133778672},
    "convT_2stage#0": {"src": "47c330d902d0d16e", "fetch_bytes": 141292053, "write_bytes": 1352989936},
    "convT_2stage#1": {"src": "47c330d902d0d16e", "fetch_bytes": 1223667009, "write_bytes": 1121198160},
}
KERNEL_SOURCES = {
    "conv": ["conv_pool.hip", "ps_internal.h"],
    "conv_bf16": ["conv_pool.hip", "ps_internal.h"],
    "maxpool": ["maxpool.hip", "ps_internal.h"],
    "convT": ["convt_softmax.hip", "convt_rows.hip", "ps_internal.h"],
    "conv_general": ["conv_general.hip", "ps_internal.h"],
    "convT_bf16": ["convt_softmax_bf16.hip", "convt_rows.hip", "ps_internal.h"],
    "maxpool_s2": ["maxpool.hip", "ps_internal.h"],
    "maxpool_d2": ["maxpool.hip", "ps_internal.h"],
    "conv_2stage": ["conv_general.hip", "two_stage.hip", "ps_internal.h"],
    "convT_2stage": ["convt_softmax.hip", "convt_rows.hip", "two_stage.hip", "ps_internal.h"],
}


def source_hash(op):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[op]:
        with open(os.path.join(ROOT, "pool_stencil_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(op):
    """HBM bytes per launch of `op` (a stage of a two-stage op is "name#i"), or None."""
    t = TRAFFIC.get(op)
    if not t or t["src"] != source_hash(op.split("#")[0]):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing and the clock probe (profiling runs)")
    ap.add_argument("--ops",
                    default="conv,maxpool,convT,conv_bf16,conv_general,convT_bf16,maxpool_s2,"
                            "maxpool_d2,conv_2stage,convT_2stage,tiny_conv")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a 2 GiB device-to-device copy instead (counter calibration)")
    return ap.parse_args()


def copy_calibration(steps):
    """A plain device copy of known size: 2 GiB read + 2 GiB written per launch."""
    import torch
    n = 32 * 64 * 512 * 512
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_calibration": True, "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": ms, "GBps": 2 * n * 4 / ms / 1e6}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the operations shard over the batch with no communication, so the one-GPU "
              "figure is the per-GPU figure", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    # the clock probe's helper starts before anything here touches the GPU (profiling
    # runs skip it)
    helper = None if args.no_cpu_baseline else start_clock_helper()

    import numpy as np
    import torch

    import inputgen
    import pool_stencil_amd as ps

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops = [o for o in args.ops.split(",") if o]
    t0 = time.time()

    def put(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            t = t.view(dtype)
        return t.to(dev)

    runs = {}
    if "conv" in ops:
        c = inputgen.workload("conv")
        xd, wd, cb, b2 = put(c["x"]), put(c["w"]), put(c["conv_bias"]), put(c["bias2"])
        out = torch.empty((128, 64, 63, 63), dtype=torch.float32, device=dev)
        runs["conv"] = lambda xd=xd, wd=wd, cb=cb, b2=b2, out=out: ps.conv_tanh_scale_bias_maxpool(
            xd, wd, cb, b2, 2.0, 4, out=out)
        del c
    if any(o in ops for o in ("maxpool", "maxpool_s2", "maxpool_d2")):
        c = inputgen.workload("maxpool")
        xp = put(c["x"])
        del c
    if "maxpool" in ops:
        outp = torch.empty((32, 64, 511, 511), dtype=torch.float32, device=dev)
        runs["maxpool"] = lambda xp=xp, outp=outp: ps.maxpool2d(xp, 4, 1, 1, 1, out=outp)
    if "maxpool_s2" in ops:
        outs2 = torch.empty((32, 64, 256, 256), dtype=torch.float32, device=dev)
        runs["maxpool_s2"] = lambda xp=xp, outs2=outs2: ps.maxpool2d(xp, 3, 2, 1, 1, out=outs2)
    if "maxpool_d2" in ops:
        outd2 = torch.empty((32, 64, 512, 512), dtype=torch.float32, device=dev)
        runs["maxpool_d2"] = lambda xp=xp, outd2=outd2: ps.maxpool2d(xp, 3, 1, 2, 2, out=outd2)
    if "convT" in ops:
        c = inputgen.workload("convT")
        xt, wt, cbt, b2t = put(c["x"]), put(c["w"]), put(c["convT_bias"]), put(c["bias2"])
        outt = torch.empty((128, 128, 129, 129), dtype=torch.float32, device=dev)
        runs["convT"] = lambda xt=xt, wt=wt, cbt=cbt, b2t=b2t, outt=outt: (
            ps.convT_softmax_bias_scale_sigmoid(xt, wt, cbt, b2t, 2.0, 2, 1, 1, 1, out=outt))
        del c
    if "conv_bf16" in ops:
        c = inputgen.workload("conv_bf16")
        xb = put(c["x_bits"].view(np.int16)).view(torch.bfloat16)
        wb = put(c["w_bits"].view(np.int16)).view(torch.bfloat16)
        cbb, b2b = put(c["conv_bias"]), put(c["bias2"])
        outb = torch.empty((128, 64, 63, 63), dtype=torch.bfloat16, device=dev)
        runs["conv_bf16"] = lambda xb=xb, wb=wb, cbb=cbb, b2b=b2b, outb=outb: (
            ps.conv_tanh_scale_bias_maxpool(xb, wb, cbb, b2b, 2.0, 4, out=outb))
        del c
    if "conv_general" in ops:
        c = inputgen.workload("conv_general")
        xg, wg, cbg, b2g = put(c["x"]), put(c["w"]), put(c["conv_bias"]), put(c["bias2"])
        outg = torch.empty((32, 128, 64, 64), dtype=torch.float32, device=dev)
        runs["conv_general"] = lambda xg=xg, wg=wg, cbg=cbg, b2g=b2g, outg=outg: (
            ps.conv_tanh_scale_bias_maxpool(xg, wg, cbg, b2g, 2.0, 3, 2, 1, 1, 1, 1, 1, out=outg))
        del c
    if "convT_bf16" in ops:
        c = inputgen.workload("convT_bf16")
        xtb = put(c["x_bits"].view(np.int16)).view(torch.bfloat16)
        wtb = put(c["w_bits"].view(np.int16)).view(torch.bfloat16)
        cbtb, b2tb = put(c["convT_bias"]), put(c["bias2"])
        outtb = torch.empty((128, 128, 129, 129), dtype=torch.bfloat16, device=dev)
        runs["convT_bf16"] = lambda xtb=xtb, wtb=wtb, cbtb=cbtb, b2tb=b2tb, outtb=outtb: (
            ps.convT_softmax_bias_scale_sigmoid(xtb, wtb, cbtb, b2tb, 2.0, 2, 1, 1, 1, out=outtb))
        del c
    if "tiny_conv" in ops:
        c = inputgen.workload("tiny_conv")
        xs, ws, cbs, b2s = put(c["x"]), put(c["w"]), put(c["conv_bias"]), put(c["bias2"])
        outs = torch.empty((2, 16, 7, 7), dtype=torch.float32, device=dev)
        runs["tiny_conv"] = lambda xs=xs, ws=ws, cbs=cbs, b2s=b2s, outs=outs: (
            ps.conv_tanh_scale_bias_maxpool(xs, ws, cbs, b2s, 2.0, 4, out=outs))
        del c
    stages = {}   # op -> list of stage callables (timed one by one)
    if "conv_2stage" in ops:
        c = inputgen.workload("conv")
        x2, w2, cb2, b22 = put(c["x"]), put(c["w"]), put(c["conv_bias"]), put(c["bias2"])
        inter = torch.empty((128, 64, 254, 254), dtype=torch.float32, device=dev)
        out2 = torch.empty((128, 64, 63, 63), dtype=torch.float32, device=dev)
        stages["conv_2stage"] = [
            lambda x2=x2, w2=w2, cb2=cb2, inter=inter: ps.conv2d(x2, w2, cb2, out=inter),
            lambda inter=inter, b22=b22, out2=out2: ps.tanh_scale_bias_maxpool(
                inter, b22, 2.0, 4, out=out2)]
        del c
    if "convT_2stage" in ops:
        c = inputgen.workload("convT")
        xt2, wt2, cbt2, b2t2 = put(c["x"]), put(c["w"]), put(c["convT_bias"]), put(c["bias2"])
        intert = torch.empty((128, 128, 129, 129), dtype=torch.float32, device=dev)
        stages["convT_2stage"] = [
            lambda xt2=xt2, wt2=wt2, cbt2=cbt2, intert=intert: ps.convT2d(
                xt2, wt2, cbt2, 2, 1, 1, 1, out=intert),
            lambda intert=intert, b2t2=b2t2: ps.softmax_bias_scale_sigmoid(
                intert, b2t2, 2.0, out=intert)]
        del c
    for name, fns in stages.items():
        for si, fn in enumerate(fns):
            runs[f"{name}#{si}"] = fn
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s; ops {list(runs)}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        for name, fn in runs.items():
            fn()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    ev = {name: [] for name in runs}
    step_start = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_start.record()
    for i in range(args.steps):
        for name, fn in runs.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
    step_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = step_start.elapsed_time(step_end)
    ms = {name: [a.elapsed_time(b) for a, b in pairs] for name, pairs in ev.items()}
    print(f"[bench] timed {args.steps} steps in {wall:.2f}s", file=sys.stderr, flush=True)

    def stats(name):
        v = np.array(ms[name])
        return float(v.mean()), float(np.median(v)), float(v.min())

    out_ops = {}
    if "conv" in runs:
        mean, med, mn = stats("conv")
        ach = CONV_FLOP / (mean * 1e-3)
        out_ops["conv"] = {
            "value": ach / 1e9, "unit": "GFLOP/s", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gflop_per_launch": CONV_FLOP / 1e9,
            "value_page_count": CONV_FLOP_PAGE / (mean * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": ach / 1e12, "peak": PEAK_FP32 / 1e12,
                         "unit": "TFLOP/s", "frac": ach / PEAK_FP32, "traffic": traffic("conv")}}
    if "maxpool" in runs:
        mean, med, mn = stats("maxpool")
        ach = POOL_BYTES / (mean * 1e-3)
        out_ops["maxpool"] = {
            "value": ach / 1e9, "unit": "GB/s", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gbytes_per_launch": POOL_BYTES / 1e9,
            "roofline": {"bound": "hbm", "achieved": ach / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": ach / PEAK_HBM, "traffic": traffic("maxpool")}}
    if "convT" in runs:
        mean, med, mn = stats("convT")
        ach = CONVT_FLOP / (mean * 1e-3)
        out_ops["convT"] = {
            "value": ach / 1e9, "unit": "GFLOP/s", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gflop_per_launch": CONVT_FLOP / 1e9,
            "hbm_GBps": CONVT_BYTES / (mean * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": ach / 1e12, "peak": PEAK_FP32 / 1e12,
                         "unit": "TFLOP/s", "frac": ach / PEAK_FP32, "traffic": traffic("convT")}}
    if "conv_bf16" in runs:
        mean, med, mn = stats("conv_bf16")
        ach = CONV_FLOP / (mean * 1e-3)
        out_ops["conv_bf16"] = {
            "value": ach / 1e9, "unit": "GFLOP/s", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gflop_per_launch": CONV_FLOP / 1e9,
            "roofline": {"bound": "mfma", "achieved": ach / 1e12, "peak": PEAK_BF16 / 1e12,
                         "unit": "TFLOP/s", "frac": ach / PEAK_BF16, "traffic": traffic("conv_bf16"),
                         "frac_of_fp32_peak": ach / PEAK_FP32}}

    if "conv_general" in runs:
        mean, med, mn = stats("conv_general")
        ach = CONV_GENERAL_FLOP / (mean * 1e-3)
        out_ops["conv_general"] = {
            "value": ach / 1e9, "unit": "GFLOP/s", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gflop_per_launch": CONV_GENERAL_FLOP / 1e9,
            "roofline": {"bound": "mfma", "achieved": ach / 1e12, "peak": PEAK_FP32 / 1e12,
                         "unit": "TFLOP/s", "frac": ach / PEAK_FP32,
                         "traffic": traffic("conv_general")}}

    for name, nbytes in (("maxpool_s2", POOL_S2_BYTES), ("maxpool_d2", POOL_D2_BYTES)):
        if name in runs:
            mean, med, mn = stats(name)
            ach = nbytes / (mean * 1e-3)
            out_ops[name] = {
                "value": ach / 1e9, "unit": "GB/s", "ms_mean": mean, "ms_median": med,
                "ms_min": mn, "gbytes_per_launch": nbytes / 1e9,
                "roofline": {"bound": "hbm", "achieved": ach / 1e9, "peak": PEAK_HBM / 1e9,
                             "unit": "GB/s", "frac": ach / PEAK_HBM, "traffic": traffic(name)}}
    if "convT_bf16" in runs:
        mean, med, mn = stats("convT_bf16")
        bw = CONVT_BF16_BYTES / (mean * 1e-3)
        out_ops["convT_bf16"] = {
            "value": CONVT_FLOP / (mean * 1e-3) / 1e9, "unit": "GFLOP/s", "ms_mean": mean,
            "ms_median": med, "ms_min": mn, "gflop_per_launch": CONVT_FLOP / 1e9,
            "frac_of_bf16_peak": CONVT_FLOP / (mean * 1e-3) / PEAK_BF16,
            "roofline": {"bound": "hbm", "achieved": bw / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": bw / PEAK_HBM, "traffic": traffic("convT_bf16")}}
    if "conv_2stage#0" in runs:
        m0, m1 = stats("conv_2stage#0")[0], stats("conv_2stage#1")[0]
        a0 = CONV_FLOP_PAGE / (m0 * 1e-3)
        b1 = (CONV_INTER_BYTES + 128 * 64 * 63 * 63 * 4) / (m1 * 1e-3)
        fused = out_ops.get("conv", {}).get("ms_mean")
        out_ops["conv_2stage"] = {
            "value": CONV_FLOP / ((m0 + m1) * 1e-3) / 1e9, "unit": "GFLOP/s",
            "ms_mean": m0 + m1, "stage_ms": [m0, m1],
            "fusion_speedup": (m0 + m1) / fused if fused else None,
            "roofline": {"bound": "mfma", "achieved": a0 / 1e12, "peak": PEAK_FP32 / 1e12,
                         "unit": "TFLOP/s", "frac": a0 / PEAK_FP32,
                         "traffic": traffic("conv_2stage#0"),
                         "kernel": "conv2d stage (76.1 GFLOP over all 254x254 outputs)"},
            "stage2_roofline": {"bound": "hbm", "achieved": b1 / 1e9, "peak": PEAK_HBM / 1e9,
                                "unit": "GB/s", "frac": b1 / PEAK_HBM,
                                "traffic": traffic("conv_2stage#1")}}
    if "convT_2stage#0" in runs:
        m0, m1 = stats("convT_2stage#0")[0], stats("convT_2stage#1")[0]
        a0 = CONVT_FLOP / (m0 * 1e-3)
        b1 = 2 * CONVT_INTER_BYTES / (m1 * 1e-3)
        fused = out_ops.get("convT", {}).get("ms_mean")
        out_ops["convT_2stage"] = {
            "value": CONVT_FLOP / ((m0 + m1) * 1e-3) / 1e9, "unit": "GFLOP/s",
            "ms_mean": m0 + m1, "stage_ms": [m0, m1],
            "fusion_speedup": (m0 + m1) / fused if fused else None,
            "roofline": {"bound": "mfma", "achieved": a0 / 1e12, "peak": PEAK_FP32 / 1e12,
                         "unit": "TFLOP/s", "frac": a0 / PEAK_FP32,
                         "traffic": traffic("convT_2stage#0"), "kernel": "convT stage"},
            "stage2_roofline": {"bound": "hbm", "achieved": b1 / 1e9, "peak": PEAK_HBM / 1e9,
                                "unit": "GB/s", "frac": b1 / PEAK_HBM,
                                "traffic": traffic("convT_2stage#1")}}

    if "tiny_conv" in runs:
        mean, med, mn = stats("tiny_conv")
        out_ops["tiny_conv"] = {
            "value": mean * 1e3, "unit": "us", "ms_mean": mean, "ms_median": med, "ms_min": mn,
            "gflops": TINY_FLOP / (mean * 1e-3) / 1e9,
            "roofline": None, "note": "launch-latency bound (3.61 MFLOP): no roofline claim"}

    # GPU clocks while the fused conv runs, and a plain device copy as a practical HBM
    # ceiling (outside the timed step)
    clocks = sample_clocks(helper, runs.get("conv"))
    gpu_info = {"clocks_during_conv": clocks, "hbm_copy": copy_ceiling()}
    sclk = mhz(clocks, "sclk clock speed")
    if sclk:
        # the published 157.3 TFLOP/s is 256 CUs x 2.4 GHz x 256 fp32 FLOP per clock per CU
        ncu = torch.cuda.get_device_properties(dev).multi_processor_count
        gpu_info["fp32_peak_at_observed_sclk_TFLOPs"] = ncu * sclk * 1e6 * 256 / 1e12
    head = "conv" if "conv" in out_ops else next(iter(out_ops))
    cpu = None
    host = host_info()
    if not args.no_cpu_baseline:
        for op in CPU_SAMPLES:
            if op in out_ops:
                out_ops[op]["cpu_baseline"] = cpu_baseline(op, host)
                print(f"[bench] cpu baseline {op}: {out_ops[op]['cpu_baseline']['seconds']:.2f}s",
                      file=sys.stderr, flush=True)
        cpu = out_ops[head].get("cpu_baseline")

    line = {
        "metric": "fused conv+maxpool GFLOP/s & maxpool GB/s, % of MI355X roofline, 1 GPU",
        "value": out_ops[head]["value"],
        "unit": out_ops[head]["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "conv2d 8->64 k3 + tanh + *2 + bias + maxpool4, x fp32 [128,8,256,256] "
                        "-> [128,64,63,63]",
            "step": list(runs),
            "maxpool_workload": "maxpool2d k4 s1 p1 d1, x fp32 [32,64,512,512] -> [32,64,511,511]",
            "convT_workload": "convT 64->128 k4 s2 p1 op1 + softmax(c) + bias + *2 + sigmoid, "
                              "x fp32 [128,64,64,64] -> [128,128,129,129]",
            "conv_bf16_workload": "conv workload with bf16 x/w/out, fp32 accumulate",
            "conv_general_workload": "conv2d 64->128 k3 p1 + tanh + *2 + bias + maxpool k3 s2 p1, "
                                     "x fp32 [32,64,128,128] -> [32,128,64,64]",
            "convT_bf16_workload": "convT workload with bf16 x/w/out, fp32 accumulate",
            "maxpool_s2_workload": "maxpool2d k3 s2 p1 on the maxpool input -> [32,64,256,256]",
            "maxpool_d2_workload": "maxpool2d k3 s1 p2 d2 on the maxpool input -> [32,64,512,512]",
            "two_stage": "conv_2stage / convT_2stage: the conv and convT workloads unfused "
                         "(intermediate stored in HBM), for the fusion comparison",
        },
        "roofline": out_ops[head]["roofline"],
        "cpu_baseline": cpu,
        "maxpool_GBps": out_ops.get("maxpool", {}).get("value"),
        "host": host,
        "gpu": gpu_info,
        "ops": out_ops,
    }
    print(json.dumps(line), flush=True)


def host_info():
    """CPU model, the cores this process may run on, and the oracle's OpenMP threads."""
    import oracle
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "omp_threads": oracle.num_threads()}


CLOCK_HELPER = r"""
import subprocess, sys
for _ in sys.stdin:
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        out = r.stdout
    except Exception as e:
        out = ""
    sys.stdout.write(out.replace(chr(10), " ") + chr(10))
    sys.stdout.flush()
"""


def start_clock_helper():
    """A helper process that runs rocm-smi on request.  It is started before this
    process touches the GPU, so neither it nor the rocm-smi it starts inherits an
    initialised GPU runtime."""
    import subprocess
    try:
        return subprocess.Popen([sys.executable, "-c", CLOCK_HELPER], stdin=subprocess.PIPE,
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def sample_clocks(helper, fn, seconds=20.0):
    """rocm-smi's current clocks, read while `fn` (the fused conv) runs back to back."""
    import threading
    import torch
    if helper is None or fn is None:
        return None
    reply = []
    helper.stdin.write("go\n")
    helper.stdin.flush()
    reader = threading.Thread(target=lambda: reply.append(helper.stdout.readline()), daemon=True)
    reader.start()
    t0 = time.perf_counter()
    while reader.is_alive() and time.perf_counter() - t0 < seconds:
        for _ in range(200):
            fn()
        torch.cuda.synchronize()
    helper.stdin.close()
    try:
        data = json.loads(reply[0]) if reply else None
    except ValueError:
        data = None
    if not isinstance(data, dict) or not data:
        return None
    card = next(iter(data.values()))
    return {k.rstrip(":"): v for k, v in card.items() if "clock" in k.lower()}


def mhz(clocks, key):
    """The MHz figure of a rocm-smi clock entry such as '(2342Mhz)', or None."""
    import re
    if not isinstance(clocks, dict) or key not in clocks:
        return None
    m = re.search(r"([0-9.]+)\s*mhz", str(clocks[key]), re.I)
    return float(m.group(1)) if m else None


def copy_ceiling(steps=10):
    """A device-to-device copy of 1 GiB (read + write), the practical ceiling of a
    mixed read/write stream on this GPU."""
    import torch
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del x, y
    torch.cuda.empty_cache()
    return {"bytes_per_copy": 2 * 4 * n, "ms": ms, "GBps": 2 * 4 * n / (ms * 1e-3) / 1e9,
            "what": "torch device copy of 1 GiB (1 GiB read + 1 GiB written)"}


# op -> (workload, images in the sample, algorithmic work of the sample, unit)
CPU_SAMPLES = {
    "conv": ("conv", 128, CONV_FLOP, "GFLOP/s"),
    "conv_bf16": ("conv_bf16", 128, CONV_FLOP, "GFLOP/s"),
    "maxpool": ("maxpool", 32, POOL_BYTES, "GB/s"),
    "maxpool_s2": ("maxpool", 32, POOL_S2_BYTES, "GB/s"),
    "maxpool_d2": ("maxpool", 32, POOL_D2_BYTES, "GB/s"),
    "convT": ("convT", 32, CONVT_FLOP / 4, "GFLOP/s"),
    "convT_bf16": ("convT_bf16", 32, CONVT_FLOP / 4, "GFLOP/s"),
    "conv_general": ("conv_general", 8, CONV_GENERAL_FLOP / 4, "GFLOP/s"),
    "tiny_conv": ("tiny_conv", 2, TINY_FLOP, "us"),
}
POOL_ARGS = {"maxpool": (4, 1, 1, 1), "maxpool_s2": (3, 2, 1, 1), "maxpool_d2": (3, 1, 2, 2)}


def cpu_baseline(op, host):
    """The oracle (plain C, fp64, OpenMP) on a bounded slice of the op's workload, in
    the op's unit, counted with the same algorithmic work as the GPU figure."""
    import oracle
    import inputgen
    name, n_img, work, unit = CPU_SAMPLES[op]
    c = inputgen.workload(name)
    total = c["N"]
    if op in POOL_ARGS:
        x = c["x"][:n_img]
        t = time.perf_counter()
        oracle.maxpool2d(x, *POOL_ARGS[op])
        dt = time.perf_counter() - t
        what = f"max-pool of the first {n_img} of {total} images, float32 (exact)"
    else:
        c1 = dict(c, x=c["x"][:n_img], N=n_img)
        fn = (oracle.convT_softmax_bias_scale_sigmoid if name.startswith("convT")
              else oracle.conv_tanh_scale_bias_maxpool)
        reps = 200 if op == "tiny_conv" else 1
        t = time.perf_counter()
        for _ in range(reps):
            fn(c1)
        dt = (time.perf_counter() - t) / reps
        what = (f"the first {n_img} of {total} images of the {name} workload, the full fused "
                f"op in written order, double precision")
    value = dt * 1e6 if unit == "us" else work / dt / 1e9   # GB/s or GFLOP/s
    return {"value": value, "unit": unit, "cores": host["omp_threads"], "kind": "oracle",
            "seconds": dt, "sample": what + "; work counted as for the GPU figure",
            "cpu_model": host["cpu_model"], "affinity_cores": host["affinity_cores"]}


if __name__ == "__main__":
    main()
