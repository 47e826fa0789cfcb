"""Benchmark of the ConvTranspose forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one convt_forward call (weight reorder, for the two-byte GEMM together
with the input's channel-chunked copy in one launch, then the main kernel) on one batch
of seeded synthetic input already resident in HBM. Steps rotate over enough
buffer sets (x, W, bias, y, workspace) that their total exceeds the 256 MB
Infinity Cache, so each step reads its inputs from HBM rather than from a
cache warmed by the previous step. The default workload is the largest
single-GPU configuration, the 2-D bfloat16 generator upsampling
x[64,512,16,16] W[512,256,4,4] stride 2 pad 1 bias[256] (68.7 GFLOP per step);
--workload selects the others.

Printed: one JSON line with the useful-FLOP throughput (2*B*C_in*(C_out/g)*
prod(k)*prod(I) per step / seconds per step), the roofline of the dominant
kernel (its average duration measured live with HIP events on the stream it
runs on) and the CPU oracle's throughput on a bounded sample of the same
workload (a reported baseline, not a target). A "backward_data" object adds
the input-gradient pass (convt_backward_data) on the same workload, timed
the same way outside the forward steps (--no-backward skips it).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

import workloads

DEFAULT_WORKLOAD = "c3_2d_bf16_generator"

# MI355X published dense peaks: 256 CUs at 2.4 GHz; bf16/f16 MFMA 4096 flop per
# clock per CU (2516.6 TFLOP/s), fp32 MFMA 256 (157.3 TFLOP/s)
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}
PEAK_HBM_GBS = 8000.0

# the source files whose change invalidates stored PMC traffic figures
KERNEL_SOURCES = {
    "phase_gemm": ["k_gemm_nchw.hip", "k_phase_gemm.hip", "kcommon.h", "convt_internal.h", "plan.cpp"],
    "phase_gemm_packed": ["k_phase_gemm.hip", "kcommon.h", "convt_internal.h", "plan.cpp"],
    "phase_gemm_allphase": ["k_gemm_allphase.hip", "kcommon.h", "convt_internal.h", "plan.cpp"],
    "grouped": ["k_grouped.hip", "kcommon.h", "plan.cpp"],
    "direct": ["k_misc.hip", "kcommon.h", "plan.cpp"],
    "naive": ["k_misc.hip", "kcommon.h", "plan.cpp"],
}
KERNEL_SYMBOL = {
    "phase_gemm": "phase_gemm_kernel",
    "phase_gemm_packed": "phase_gemm_kernel",
    "phase_gemm_allphase": "allphase_gemm_kernel",
    "grouped": "grouped_kernel",
    "direct": "direct_kernel",
    "naive": "naive_kernel",
}


def kernel_hash(route: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(route, []):
        with open(os.path.join(ROOT, "convt_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl: workloads.Workload, out_shape) -> int:
    """x + W + bias read once, y written once, in the workload's element type."""
    eb = 4 if wl.dtype == "f32" else 2
    n = int(np.prod(wl.x_shape)) + int(np.prod(wl.w_shape)) + int(np.prod(out_shape))
    if wl.has_bias:
        n += wl.c_out
    return n * eb


def useful_flops(wl: workloads.Workload) -> int:
    b, cin = wl.x_shape[0], wl.x_shape[1]
    return 2 * b * cin * wl.w_shape[1] * int(np.prod(wl.w_shape[2:])) * int(np.prod(wl.x_shape[2:]))


def stored_traffic(route: str, wl_name: str):
    """HBM bytes per launch from the committed PMC summary of this kernel and
    workload, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"{route}_{wl_name}_pmc.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"^kernel_source_sha256_16:\s*(\S+)", txt, re.M)
    m_tr = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_hash or not m_tr or m_hash.group(1) != kernel_hash(route):
        return None
    return float(m_tr.group(1))


def cpu_baseline(wl: workloads.Workload, tens: workloads.Tensors, target_s: float = 20.0):
    """The oracle (untuned) on the host cores, on a batch subset of the
    workload sized to roughly target_s seconds (at least one batch item; the
    whole batch repeated if it is faster than that)."""
    import oracle

    prm = dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation,
               output_padding=wl.output_padding, groups=wl.groups)
    flops_per_item = useful_flops(wl) / wl.x_shape[0]
    # probe with one batch item (the second call: the first also starts the
    # oracle's threads)
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.forward(tens.x[:1], tens.w, tens.bias, with_scale=False, **prm)
        t1 = time.perf_counter() - t0
    items = int(max(1, min(wl.x_shape[0], target_s / max(t1, 1e-6))))
    reps = 1
    if items == wl.x_shape[0]:
        reps = int(max(1, target_s / max(t1 * items, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.forward(tens.x[:items], tens.w, tens.bias, with_scale=False, **prm)
    dt = time.perf_counter() - t0
    flops = flops_per_item * items * reps
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{items} of {wl.x_shape[0]} batch items x {reps} pass(es), value-only fp64 "
                  f"scatter-add, {dt:.1f} s wall",
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_backward(pl, wl, sets, stream, K, warmup):
    """convt_backward_data on the same workload: dx from dy through the same
    weights, back-to-back calls over the rotating buffer sets (dy: the sets'
    forward outputs; dx overwrites their inputs), bracketed by one event
    pair on the launch stream. A call is the whole backward pass: weight
    reorder, the channel-chunked copy of dy (bfloat16) and the GEMM."""
    import torch
    dev = sets[0]["x"].device
    sh = stream.cuda_stream
    wss = [pl.new_bwd_workspace(dev) for _ in sets]

    def call(i):
        s = sets[i % len(sets)]
        pl.backward_data_ptr(s["y"].data_ptr(), s["w"].data_ptr(), s["x"].data_ptr(),
                             wss[i % len(sets)].data_ptr(), sh)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / K
    flops = useful_flops(wl)
    peak = PEAK_TFLOPS.get(wl.dtype)
    return {
        "route": pl.route_bwd,
        "us_per_call": t * 1e6,
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "frac_of_mfma_peak": flops / t / 1e12 / peak if peak else None,
        "calls": K,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="one of " + ", ".join(sorted(workloads.WORKLOADS)) + " or a short alias")
    ap.add_argument("--rotate-mb", type=float, default=1024.0,
                    help="total size of the rotated buffer sets (defeats the 256 MB cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", choices=["f32", "bf16", "f16"], default=None,
                    help="element type (default: the workload's)")
    ap.add_argument("--activation", default="none",
                    choices=["none", "relu", "sigmoid", "tanh", "silu", "gelu"],
                    help="activation fused after the bias (default none, as the workloads)")
    ap.add_argument("--route", default="auto",
                    help="force a forward route (convt_route name, e.g. phase_gemm_packed)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-data (input gradient) measurement")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (3 times), "
                         "the reference kernel for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import convt_forward_amd as C

    wl = workloads.get(args.workload)
    if args.dtype is not None and args.dtype != wl.dtype:
        import dataclasses
        wl = dataclasses.replace(wl, dtype=args.dtype)
    tens = workloads.workload_tensors(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pl = C.get_plan(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.dilation,
                    wl.output_padding, wl.groups, wl.has_bias, wl.dtype, route=args.route,
                    activation=args.activation)

    def to_dev(a):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        return t.view(torch.float16 if wl.dtype == "f16" else torch.bfloat16)

    x0, w0 = to_dev(tens.x_dev), to_dev(tens.w_dev)
    b0 = to_dev(tens.bias_dev) if wl.has_bias else None
    eb = 4 if wl.dtype == "f32" else 2
    set_bytes = (x0.numel() + w0.numel() + (b0.numel() if b0 is not None else 0) +
                 int(np.prod(pl.out_shape))) * eb + pl.workspace_bytes
    nsets = int(max(1, min(256, np.ceil(args.rotate_mb * 1e6 / set_bytes))))
    sets = []
    for i in range(nsets):
        sets.append(dict(x=x0 if i == 0 else x0.clone(), w=w0 if i == 0 else w0.clone(),
                         b=(b0 if i == 0 else b0.clone()) if b0 is not None else None,
                         y=pl.new_output(dev), ws=pl.new_workspace(dev)))
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step(s, ev0=None, ev1=None):
        # one convt_forward: weight reorder (with the input pack, for the
        # two-byte GEMM, in the same launch), then the main kernel
        if ev0 is not None:
            ev0.record(stream)
        pl.forward_ptr(s["x"].data_ptr(), s["w"].data_ptr(),
                       s["b"].data_ptr() if s["b"] is not None else 0, s["y"].data_ptr(),
                       s["ws"].data_ptr(), sh)
        if ev1 is not None:
            ev1.record(stream)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / K

    # a step's GPU time from event pairs around it (a separate pass:
    # recording events inside the timed loop would add host work to it)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(K, 50))]
    for i, (e0, e1) in enumerate(ev):
        step(sets[i % nsets], e0, e1)
    torch.cuda.synchronize()
    step_us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    step_gpu_s = float(np.mean(step_us)) / 1e6

    # The dominant kernel alone: back-to-back launches over the same rotating
    # buffer sets (weights prepared once per set), bracketed by one event
    # pair on the launch stream, so that dispatch gaps after the reorder
    # kernel are not charged to it. At least 400 launches: under sustained
    # MFMA load the part's clock moves over the first milliseconds (a short
    # fast stretch of about 20 launches of the generator workload's kernel,
    # a slower one of several tens, then steady), so a pass of 100 launches
    # measured whichever stretch it fell in (about 69 us per launch when it
    # started after 105 launches, 75 us after 45); 400 launches span the
    # slow stretch and the steady state that sustained use runs in.
    for s in sets:
        pl.prepare_weights_ptr(s["w"].data_ptr(), s["ws"].data_ptr(), sh)
    torch.cuda.synchronize()
    KK = max(K, 400)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(KK):
        s = sets[i % nsets]
        pl.forward_prepared_ptr(s["x"].data_ptr(), s["w"].data_ptr(),
                                s["b"].data_ptr() if s["b"] is not None else 0, s["y"].data_ptr(),
                                s["ws"].data_ptr(), sh)
    k1.record(stream)
    torch.cuda.synchronize()
    kern_s = k0.elapsed_time(k1) / 1e3 / KK

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = useful_flops(wl)
    abytes = algorithmic_bytes(wl, pl.out_shape)
    route = pl.route
    if route in ("phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "direct", "naive") and \
            wl.dtype in PEAK_TFLOPS and \
            flops / abytes > 50.0:
        bound, unit = "mfma", "TFLOP/s"
        achieved = flops / kern_s / 1e12
        peak = PEAK_TFLOPS[wl.dtype]
    else:
        bound, unit = "hbm", "GB/s"
        achieved = abytes / kern_s / 1e9
        peak = PEAK_HBM_GBS
    traffic = stored_traffic(route, wl.name)
    kernel = KERNEL_SYMBOL.get(route, route)
    if route == "phase_gemm" and wl.dtype != "f32":
        kernel = "phase_gemm_nchw_kernel"
    if route == "phase_gemm_packed":
        # the packed GEMM reads a channel-chunked copy of x that a pack
        # kernel writes inside the same forward call: kernel_us covers both
        kernel = "pack_x_kernel+phase_gemm_kernel"
    roofline = {
        "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
        "frac": achieved / peak, "traffic": traffic,
        "kernel": kernel, "kernel_us": kern_s * 1e6, "kernel_launches": KK,
        "step_us_events": step_gpu_s * 1e6,
        "step_us_events_median": float(np.median(step_us)),
        "step_us_events_min": float(np.min(step_us)),
        "algorithmic_flops": flops, "algorithmic_bytes": abytes,
        "kernel_source_sha256_16": kernel_hash(route),
    }

    result = {
        "metric": "useful TFLOP/s (2*B*Cin*Cout/g*taps*in_spatial)",
        "value": flops / sec_per_step / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "ms_per_step_median": float(np.median(step_us)) / 1e3,
        "ms_per_step_min": float(np.min(step_us)) / 1e3,
        "timing": ("ms_per_step (and value): K steps back to back on the host clock, synchronized "
                   "before and after; ms_per_step_median / _min: single steps between event pairs "
                   "in a separate pass, each without the overlap of its neighbours' launches"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "x_shape": list(wl.x_shape), "w_shape": list(wl.w_shape),
            "stride": list(wl.stride), "padding": list(wl.padding),
            "dilation": list(wl.dilation), "output_padding": list(wl.output_padding),
            "groups": wl.groups, "bias": wl.has_bias, "activation": args.activation,
            "out_shape": list(pl.out_shape),
            "route": route, "buffer_sets": nsets,
            "algorithmic_GBps_per_step": abytes / sec_per_step / 1e9,
        },
        "roofline": roofline,
    }
    if not args.no_backward and pl.route_bwd != "none":
        result["backward_data"] = measure_backward(pl, wl, sets, stream, K, args.warmup)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, tens)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
