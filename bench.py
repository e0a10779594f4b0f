#!/usr/bin/env python3
"""Benchmark of conv2d grad_input on one MI355X: effective TFLOP/s and the
fraction of the matrix-core roofline, with the CPU oracle timed beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-others]

A step is one grad_input call (prologue + main kernel) over one batch of
synthetic inputs already resident in HBM.  After a device synchronize: at
least W untimed steps (and at least 0.1 s of GPU work, so the clocks have
settled), then exactly K steps timed between two events on the launch
stream, enqueued back to back with the warm-up (no idle gap before them),
then a device synchronize; rank 0 prints ONE JSON line.  Effective work per
call is 2*N*Co*oH*oW*Ci*kH*kW flops.

The main kernel's own duration is measured live with HIP events that its
launch records with the dispatch's start and end timestamps (the
``roofline.achieved`` figure); the whole-call time gives ``value``.
``roofline.traffic`` is the HBM bytes per launch from the committed counter
summary under profiles/, and ``roofline.mfma_counters`` the matrix-core work
and utilisation the MFMA counters saw per launch, each when its kernel
sources and plan still match.

Beside the warm figure, every workload is also timed cold: before each of
``--cold-steps`` calls a 512 MiB device buffer is overwritten (more than the
L2s and the 256 MB last-level cache hold), and each call is bracketed by its
own events; the line reports their median, min and max.  The matrix-core
peaks are measured too (a probe kernel of back-to-back MFMAs on varied data)
and each roofline fraction is given against both the published and the
measured peak.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from conv2d_backward_amd import profiling  # noqa: E402

METRIC = "effective TFLOP/s of conv2d grad_input per config; % of MFMA peak (1 GPU)"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}   # MI355X dense matrix-core peaks
PLAN_KIND = {"f32": 0, "bf16": 1, "f16": 2}   # the dtype argument of the plan description
HBM_PEAK_GBS = 8000.0
EVICT_MIB = 512        # written before each cold call: > L2s (8 x 4 MB) + 256 MB MALL
DEFAULT_WORKLOAD = "resnet_stage_3x3"
WARMUP_SECONDS = 0.1   # untimed warm-up: at least this much GPU work


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--op", default="grad_input",
                    choices=["grad_input", "grad_weight", "backward", "forward"],
                    help="the operation of the headline line (grad_weight: fp32 workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the short timing of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="calls timed one by one after evicting the caches (0: skip)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="end with %d plain device copies of this many MiB (the "
                         "reference kernel for scaling HBM byte counters)"
                         % profiling.CALIBRATION_COPIES)
    return ap.parse_args()


def device_inputs(wl, torch, dev):
    g, w = workloads.make_inputs(wl)
    if wl.dtype in ("bf16", "f16"):
        t16 = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        tg = torch.from_numpy(g.view(np.int16)).to(dev).view(t16)
        tw = torch.from_numpy(w.view(np.int16)).to(dev).view(t16)
    else:
        tg = torch.from_numpy(g).to(dev)
        tw = torch.from_numpy(w).to(dev)
    out = torch.empty(wl.shape.dst_shape, dtype=torch.float32, device=dev)
    return (g, w), tg, tw, out


class HipEvents:
    """Raw HIP events (libamdhip64 via ctypes): the library records them itself
    on its launch stream, which torch.cuda.Event (created lazily) cannot see."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreate(self.ct.byref(ev))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return ev

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def time_workload(wl, steps, warmup, torch, gi, dev, op="grad_input"):
    """Returns dict with whole-call ms, main-kernel ms (HIP events), flops.

    Everything from the warm-up to the last timed call is enqueued without a
    host synchronisation in between: an idle GPU lowers its clocks within
    milliseconds, so a pause right before the timed calls would time the
    clock ramp instead of the calls.  Both timed loops are bracketed by
    events on the launch stream, and the host synchronises before the
    warm-up and after the last loop.
    """
    s = wl.shape
    _, tg, tw, out = device_inputs(wl, torch, dev)
    stream = torch.cuda.current_stream(dev)
    if op == "grad_weight":
        tx = torch.from_numpy(workloads.make_forward_input(wl)).to(dev)
        dw = torch.empty(s.weight_shape, dtype=torch.float32, device=dev)

        def call():
            gi.grad_weight(tg, tx, stride=s.stride, padding=(s.pad_h, s.pad_w),
                           kernel_hw=(s.kH, s.kW), out=dw, stream=stream)
    elif op == "forward":
        tx = torch.from_numpy(workloads.make_forward_input(wl)).to(dev)
        y = torch.empty(s.grad_out_shape, dtype=torch.float32, device=dev)

        def call():
            gi.forward(tx, tw, stride=s.stride, padding=(s.pad_h, s.pad_w), out=y,
                       stream=stream)
    elif op == "backward":
        # dx, dw and db in one library call (its main-kernel events bracket
        # the last main kernel, grad_weight's).
        tx = torch.from_numpy(workloads.make_forward_input(wl)).to(dev)
        dw = torch.empty(s.weight_shape, dtype=torch.float32, device=dev)
        db = torch.empty((s.Co,), dtype=torch.float32, device=dev)

        def call():
            gi.backward(tg, tx, tw, stride=s.stride, padding=(s.pad_h, s.pad_w),
                        kernel_hw=(s.kH, s.kW), want_db=True, dx=out, dw=dw, db=db,
                        stream=stream)
    else:
        def call():
            gi.grad_input(tg, tw, stride=s.stride, padding=(s.pad_h, s.pad_w),
                          input_hw=(s.H, s.W), out=out, stream=stream)

    hev = HipEvents()
    sp = stream.cuda_stream
    # Size the warm-up: at least W calls and at least WARMUP_SECONDS of GPU
    # work, from the GPU time of 10 probe calls (taken on a cooler GPU, so an
    # upper bound of the per-call time).
    t0, t1 = hev.create(), hev.create()
    torch.cuda.synchronize()
    hev.hip.hipEventRecord(t0, sp)
    for _ in range(10):
        call()
    hev.hip.hipEventRecord(t1, sp)
    torch.cuda.synchronize()
    per_call = max(hev.elapsed_ms(t0, t1) * 1e-3 / 10, 1e-6)
    n_warm = int(min(max(warmup, math.ceil(WARMUP_SECONDS / per_call)), 20000))
    kb = [hev.create() for _ in range(steps)]
    ke = [hev.create() for _ in range(steps)]
    wall0 = time.perf_counter()
    for _ in range(n_warm):
        call()
    # Whole calls: exactly K steps between two events, nothing else recorded.
    hev.hip.hipEventRecord(t0, sp)
    for _ in range(steps):
        call()
    hev.hip.hipEventRecord(t1, sp)
    # Main kernel alone: the library's main launch records a begin/end event
    # pair with the dispatch's own timestamps.
    for i in range(steps):
        gi.set_profile_events(kb[i], ke[i])
        call()
    gi.set_profile_events(None, None)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    total_ms = hev.elapsed_ms(t0, t1)
    kern_ms = [hev.elapsed_ms(kb[i], ke[i]) for i in range(steps)]
    for ev in kb + ke + [t0, t1]:
        hev.destroy(ev)
    return dict(ms_per_step=total_ms / steps, kernel_ms=float(np.mean(kern_ms)),
                kernel_ms_min=float(np.min(kern_ms)), wall_ms=(wall1 - wall0) * 1e3,
                warmup_calls=n_warm,
                flops=s.eff_flops * (2 if op == "backward" else 1))


def make_call(wl, torch, gi, dev, op="grad_input"):
    """The workload's library call on device-resident inputs (a closure)."""
    s = wl.shape
    _, tg, tw, out = device_inputs(wl, torch, dev)
    stream = torch.cuda.current_stream(dev)
    if op != "grad_input":
        raise ValueError(op)

    def call():
        gi.grad_input(tg, tw, stride=s.stride, padding=(s.pad_h, s.pad_w),
                      input_hw=(s.H, s.W), out=out, stream=stream)
    return call


def time_cold(wl, steps, torch, gi, dev, evict):
    """Per-call times (ms) with the caches evicted before each call: the
    eviction write and the call are enqueued back to back (the GPU stays
    busy), and each call is bracketed by its own events."""
    call = make_call(wl, torch, gi, dev)
    call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        evict.fill_(1.0)
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
    return {"evict_mib": EVICT_MIB, "calls": steps, "median_ms": round(med, 5),
            "min_ms": round(ms[0], 5), "max_ms": round(ms[-1], 5),
            "tflops_median": round(wl.shape.eff_flops / (med * 1e-3) / 1e12, 3)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def roofline_block(flops, kernel_ms, peak, measured_peak, kernel, traffic, alg_bytes, mfma):
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "measured_peak": None if measured_peak is None else round(measured_peak, 1),
            "frac_of_measured_peak": None if not measured_peak else
            round(achieved / measured_peak, 4),
            "traffic": None if traffic is None else round(traffic["bytes"]),
            "algorithmic_bytes": alg_bytes,
            "hbm_gbs": None if traffic is None else
            round(traffic["bytes"] / (kernel_ms * 1e-3) / 1e9, 1),
            "kernel": kernel, "kernel_ms": round(kernel_ms, 5), "mfma_counters": mfma}


def cpu_baseline(wl, target_s):
    """The oracle, untuned, on a bounded sample: the first n batch items of the
    same workload (n chosen from a one-item probe to take about target_s); when
    the whole batch takes less than that, whole-batch passes repeated up to
    about target_s, so that the figure is not a fraction of a second's timing."""
    import oracle
    s = wl.shape
    g, w = workloads.make_inputs(wl)
    if wl.dtype == "bf16":
        g, w = workloads.bf16_to_f32(g), workloads.bf16_to_f32(w)
    elif wl.dtype == "f16":
        g, w = workloads.f16_to_f32(g), workloads.f16_to_f32(w)
    t = time.perf_counter()
    oracle.grad_input(g[:1], w, s.stride, (s.pad_h, s.pad_w), (s.H, s.W), with_abs=False)
    one = max(time.perf_counter() - t, 1e-4)
    n = int(max(1, min(s.N, round(target_s / one))))
    t = time.perf_counter()
    oracle.grad_input(g[:n], w, s.stride, (s.pad_h, s.pad_w), (s.H, s.W), with_abs=False)
    dt = time.perf_counter() - t
    passes = 1
    if n == s.N and dt < 0.5 * target_s:
        passes = int(max(1, min(200, round(target_s / max(dt, 1e-4)))))
        t = time.perf_counter()
        for _ in range(passes):
            oracle.grad_input(g, w, s.stride, (s.pad_h, s.pad_w), (s.H, s.W), with_abs=False)
        dt = time.perf_counter() - t
    flops = s.eff_flops * n / s.N * passes
    what = ("first %d of %d batch items" % (n, s.N) if passes == 1 else
            "%d passes over all %d batch items" % (passes, s.N))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%s of %s (fp64 direct loop, %.2f s, %s)" % (what, wl.name, dt, cpu_model()),
            "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(grad_input shards over the batch with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import conv2d_backward_amd as gi
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    gi.load_library()
    dev = torch.device("cuda:0")
    wl = workloads.BY_NAME[args.workload]
    s = wl.shape
    op = args.op
    if op != "grad_input" and wl.dtype != "f32":
        print("%s is fp32 only" % op, file=sys.stderr)
        sys.exit(2)

    r = time_workload(wl, args.steps, args.warmup, torch, gi, dev, op)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    # Matrix-core rates the chip sustains (fp16 takes the bf16 figure: the
    # same MFMA shape and rate).
    measured = {"f32": gi.mfma_peak("f32"), "bf16": gi.mfma_peak("bf16")}
    measured["f16"] = measured["bf16"]
    evict = None
    if args.cold_steps > 0 and op == "grad_input":
        evict = torch.empty(EVICT_MIB * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    params = gi.make_params(*s.as_tuple()[:10])
    if op == "grad_weight":
        plan_desc = gi.grad_weight_plan(params)
    elif op == "forward":
        plan_desc = gi.forward_plan(params)
    elif op == "backward":
        plan_desc = gi.plan(params, False) + " | " + gi.grad_weight_plan(params)
    else:
        plan_desc = gi.plan(params, PLAN_KIND[wl.dtype])
    if op == "backward":
        # Several main kernels per call: the roofline is the whole call's.
        kernel = "whole call (grad_input and grad_weight kernels, prologue, reduction)"
        kernel_ms = r["ms_per_step"]
        traffic = mfma = None
        # grad_out, x and weight read once; dx, dw and db written once.
        alg_bytes = 4 * (s.N * s.Co * s.oH * s.oW + 2 * s.N * s.Ci * s.H * s.W +
                         2 * s.Co * s.Ci * s.kH * s.kW + s.Co)
    else:
        variant = profiling.plan_variant(plan_desc)
        kernel = profiling.kernel_name(variant, wl.dtype)
        kernel_ms = r["kernel_ms"]
        if op == "grad_weight":
            # grad_out and x read once, dw written once (fp32).
            alg_bytes = 4 * (s.N * s.Co * s.oH * s.oW + s.N * s.Ci * s.H * s.W +
                             s.Co * s.Ci * s.kH * s.kW)
        else:
            alg_bytes = s.algorithmic_bytes(4 if wl.dtype == "f32" else 2)
        traffic = profiling.read_traffic(kernel, wl.name, plan_desc, variant, wl.dtype)
        mfma = profiling.read_mfma(kernel, wl.name, plan_desc, variant, wl.dtype)
    achieved = r["flops"] / (kernel_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC if op == "grad_input" else METRIC.replace(
            "grad_input", {"grad_weight": "grad_weight", "forward": "forward",
                           "backward": "backward (dx + dw + db)"}[op]),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": r["warmup_calls"],
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded PCG64: grad_out N(0,1), weight Kaiming-normal%s)"
                % (", forward input N(0,1)" if op != "grad_input" else ""),
        "config": {"workload": wl.name, "op": op, "N": s.N, "Ci": s.Ci, "Co": s.Co, "H": s.H, "W": s.W,
                   "kH": s.kH, "kW": s.kW, "stride": s.stride, "pad_h": s.pad_h,
                   "pad_w": s.pad_w, "oH": s.oH, "oW": s.oW, "eff_gflop": s.eff_flops / 1e9,
                   "plan": plan_desc},
        "roofline": dict(roofline_block(r["flops"], kernel_ms, peak, measured[wl.dtype], kernel,
                                        traffic, alg_bytes, mfma),
                         per_unit="%d*Ci*kH*kW*Co flops per output pixel (n,oh,ow)"
                                  % (4 if op == "backward" else 2),
                         units_per_launch=s.N * s.oH * s.oW),
        "frac_of_peak_whole_call": round(value / peak, 4),
        "measured_mfma_peak_tflops": {k: round(v, 1) for k, v in measured.items()},
    }
    if evict is not None:
        line["cold"] = time_cold(wl, args.cold_steps, torch, gi, dev, evict)
    if not args.no_others and op == "grad_input":
        others = {}
        for o in workloads.WORKLOADS:
            if o.name == wl.name:
                continue
            ro = time_workload(o, 20, 3, torch, gi, dev)
            v = ro["flops"] / (ro["ms_per_step"] * 1e-3) / 1e12
            so = o.shape
            po = gi.plan(gi.make_params(*so.as_tuple()[:10]), PLAN_KIND[o.dtype])
            vo = profiling.plan_variant(po)
            to = profiling.read_traffic(profiling.kernel_name(vo, o.dtype), o.name, po, vo,
                                        o.dtype)
            mo = profiling.read_mfma(profiling.kernel_name(vo, o.dtype), o.name, po, vo,
                                     o.dtype)
            others[o.name] = {"dtype": o.dtype, "tflops": round(v, 3),
                              "ms_per_call": round(ro["ms_per_step"], 5),
                              "frac_of_peak": round(v / PEAK_TFLOPS[o.dtype], 4),
                              "plan": po,
                              "roofline": roofline_block(
                                  ro["flops"], ro["kernel_ms"], PEAK_TFLOPS[o.dtype],
                                  measured[o.dtype], profiling.kernel_name(vo, o.dtype), to,
                                  so.algorithmic_bytes(4 if o.dtype == "f32" else 2), mo)}
            if evict is not None:
                others[o.name]["cold"] = time_cold(o, args.cold_steps, torch, gi, dev, evict)
        line["other_workloads"] = others
        # The next row of the same backward pass: grad_weight (fp32 runs).
        nxt = {}
        for o in workloads.WORKLOADS:
            if o.dtype != "f32" or o.name == "tiny":
                continue
            rw = time_workload(o, 20, 3, torch, gi, dev, "grad_weight")
            so = o.shape
            pw = gi.grad_weight_plan(gi.make_params(*so.as_tuple()[:10]))
            vw = rw["flops"] / (rw["ms_per_step"] * 1e-3) / 1e12
            nxt[o.name] = {"tflops": round(vw, 3), "ms_per_call": round(rw["ms_per_step"], 5),
                           "kernel_ms": round(rw["kernel_ms"], 5),
                           "frac_of_peak": round(vw / PEAK_TFLOPS["f32"], 4),
                           "kernel_frac_of_peak": round(
                               rw["flops"] / (rw["kernel_ms"] * 1e-3) / 1e12
                               / PEAK_TFLOPS["f32"], 4),
                           "plan": pw}
        # The whole backward pass of the layer in one call: dx + dw + db
        # (flops of dx and dw; the bias sums ride on the grad_weight kernel).
        bwd = {}
        for o in workloads.WORKLOADS:
            if o.dtype != "f32" or o.name == "tiny":
                continue
            rb = time_workload(o, 20, 3, torch, gi, dev, "backward")
            vb = rb["flops"] / (rb["ms_per_step"] * 1e-3) / 1e12
            bwd[o.name] = {"tflops": round(vb, 3), "ms_per_call": round(rb["ms_per_step"], 5),
                           "frac_of_peak": round(vb / PEAK_TFLOPS["f32"], 4),
                           "ms_dx_plus_dw_separately": round(
                               others.get(o.name, {}).get("ms_per_call", r["ms_per_step"]
                                                          if o.name == wl.name else float("nan"))
                               + nxt[o.name]["ms_per_call"], 5)}
        # The forward convolution of the same layer.
        fwd = {}
        for o in workloads.WORKLOADS:
            if o.dtype != "f32" or o.name == "tiny":
                continue
            rf = time_workload(o, 20, 3, torch, gi, dev, "forward")
            vf = rf["flops"] / (rf["ms_per_step"] * 1e-3) / 1e12
            fwd[o.name] = {"tflops": round(vf, 3), "ms_per_call": round(rf["ms_per_step"], 5),
                           "kernel_ms": round(rf["kernel_ms"], 5),
                           "frac_of_peak": round(vf / PEAK_TFLOPS["f32"], 4),
                           "plan": gi.forward_plan(gi.make_params(*o.shape.as_tuple()[:10]))}
        line["next_rows"] = {"grad_weight": nxt, "backward_dx_dw_db": bwd, "forward": fwd}
    if not args.no_cpu_baseline and op == "grad_input":
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * 1024 * 1024 // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(profiling.CALIBRATION_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
