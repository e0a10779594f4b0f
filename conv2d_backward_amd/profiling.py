"""Summaries of rocprofv3 output for the grad_input kernels (host-side text
processing only: nothing here touches a GPU or the library).

Two summaries are written under ``profiles/``, named for kernel and workload:

* ``<kernel>_<workload>_stats.md`` -- the ``--kernel-trace --stats`` table of
  one bench.py run, beside the kernel duration that bench.py measured live
  with HIP events in the same run;
* ``<kernel>_<workload>_traffic.txt`` -- HBM bytes per launch of the dominant
  kernel from two ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE, both in KiB per
  dispatch), each scaled by what the same counter reads for a plain
  device-to-device copy of known size run at the end of the same program;
* ``<kernel>_<workload>_mfma.txt`` -- the matrix-core work the counters saw
  per launch (SQ_INSTS_VALU_MFMA_MOPS_F32 / _BF16, in units of 512 flops,
  padded work included), the MFMA busy cycles, and the utilisation both imply
  against the kernel-trace duration of the same workload.

The traffic and MFMA files record a fingerprint of the kernel's sources and the
planner's description of the launch; bench.py reports its figure only while
both still match what it is about to run.

    python -m conv2d_backward_amd.profiling stats --run-dir D --bench-log L \
        --workload W --command "..." [--out-dir profiles]
    python -m conv2d_backward_amd.profiling traffic --fetch-dir D1 --write-dir D2 \
        --bench-log L --workload W --copy-mib M --command-fetch "..." \
        --command-write "..." [--out-dir profiles]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")

# Sources that define each main kernel (its launch parameters come from the
# planner, whose result is matched separately through the plan description).
KERNEL_SOURCES = {
    ("halo", "f32"): ["kernels_halo_f32.hip", "lds_barrier.h"],
    ("halo", "bf16"): ["kernels_halo_bf16.hip", "half_launch.h"],
    ("halo", "f16"): ["kernels_halo_bf16.hip", "half_launch.h"],
    ("stem", "f32"): ["kernels_stem_f32.hip"],
    ("col2im", "f32"): ["kernels_col2im_f32.hip"],
    ("img16", "bf16"): ["kernels_img16.hip", "half_launch.h", "lds_barrier.h"],
    ("img16", "f16"): ["kernels_img16.hip", "half_launch.h", "lds_barrier.h"],
    ("gw", "f32"): ["kernels_gw_f32.hip", "gw_common.h"],
    ("gwd", "f32"): ["kernels_gw_f32.hip", "gw_common.h"],
    ("fwd", "f32"): ["kernels_fwd_f32.hip", "fwd_common.h"],
    ("generic", "f32"): ["kernels_generic.hip", "half_launch.h"],
    ("generic", "bf16"): ["kernels_generic.hip", "half_launch.h"],
    ("generic", "f16"): ["kernels_generic.hip", "half_launch.h"],
}
COMMON_SOURCES = ["gi_common.h", "gi_launch.h"]
CALIBRATION_COPIES = 3   # copies bench.py runs for --calibration-copy-mib


def kernel_name(variant: str, dtype: str) -> str:
    """Short name of the main kernel of a plan: gi_<variant>_<dtype>."""
    return "gi_%s_%s" % (variant, dtype)


def plan_variant(plan_desc: str) -> str:
    """The plan's main kernel family: its variant, except that a 16-bit plan
    on the whole-image kernel (described as ``[image kernel ...]``) is img16."""
    if "[image kernel" in plan_desc:
        return "img16"
    return plan_desc.split()[0].split("=", 1)[1]


def fingerprint(variant: str, dtype: str) -> str:
    """sha256 (first 16 hex digits) over the kernel's source files."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[(variant, dtype)] + COMMON_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _matches(name: str, short: str) -> bool:
    """Whether kernel `name` (as the trace prints it) is the kernel `short`
    names.  fp16 inputs run the 16-bit kernels' fp16 instantiations:
    gi_halo_f16 is gi_halo_bf16<true, ...>, gi_generic_f16 gi_generic_bf16<true>;
    the image kernel is gi_img16<false, ...> for bf16 and <true, ...> for fp16."""
    if short.startswith("gi_img16_"):
        return ("gi_img16<%s" % ("true" if short.endswith("_f16") else "false")) in name
    if short.endswith("_f16"):
        return (short[:-4] + "_bf16<true") in name
    return (short + "<") in name or (short + "(") in name


def _bench_line(path: str) -> dict:
    with open(path) as fh:
        for line in reversed(fh.read().strip().splitlines()):
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    raise ValueError("no JSON line in %s" % path)


def _csv(run_dir: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(run_dir, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, run_dir))
    return hits[0]


def _unprofiled_kernel_ms(bench_log: str, workload: str, op: str = "grad_input"):
    """Main-kernel ms of `workload` for `op` in a bench.py run without the
    profiler (its headline line, one of its other_workloads or, for
    grad_weight, its next_rows), else None."""
    line = _bench_line(bench_log)
    if line["config"]["workload"] == workload and line["config"].get("op", "grad_input") == op:
        return line["roofline"]["kernel_ms"], "bench.py --steps %d --warmup %d" % (
            line["steps"], line["warmup"])
    if op == "grad_input":
        o = line.get("other_workloads", {}).get(workload)
        what = "other workloads"
    else:
        o = line.get("next_rows", {}).get(op, {}).get(workload)
        what = "next rows"
    if o is None:
        return None
    kms = o["roofline"]["kernel_ms"] if "roofline" in o else o["kernel_ms"]
    return kms, "bench.py (%s: 20 steps after at least 3 warm-up steps and 0.1 s)" % what


def write_stats(run_dir: str, bench_log: str, workload: str, command: str,
                out_dir: str = PROFILES, top: int = 8, plain_log: str = None) -> str:
    line = _bench_line(bench_log)
    plan = line["config"]["plan"]
    short = kernel_name(plan_variant(plan), line["dtype"])
    with open(_csv(run_dir, "kernel_stats.csv")) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    main = [r for r in rows if _matches(r["Name"], short)]
    if not main:
        raise ValueError("kernel %s not in %s" % (short, run_dir))
    out = os.path.join(out_dir, "%s_%s_stats.md" % (short, workload))
    rf = line["roofline"]
    with open(out, "w") as fh:
        fh.write("# %s on %s: rocprofv3 kernel-trace statistics\n\n" % (short, workload))
        fh.write("Command (from the repository root):\n\n    %s\n\n" % command)
        fh.write("Plan: `%s`\n\n" % plan)
        fh.write("| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |\n")
        fh.write("|---|---|---|---|---|---|\n")
        for r in rows[:top]:
            fh.write("| `%s` | %s | %.2f | %.2f | %.2f | %s%% |\n" % (
                r["Name"][:110], r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
        avg_us = float(main[0]["AverageNs"]) / 1e3
        fh.write("\nSame run, bench.py's own measurement (HIP events on the launch stream):\n\n")
        fh.write("- main kernel `%s`: %.2f us per launch (rocprofv3 average %.2f us, "
                 "ratio %.3f)\n" % (short, rf["kernel_ms"] * 1e3, avg_us,
                                    rf["kernel_ms"] * 1e3 / avg_us))
        if plain_log:
            u = _unprofiled_kernel_ms(plain_log, workload, line["config"].get("op", "grad_input"))
            if u is not None:
                fh.write("- without the profiler (`python3 %s`): %.2f us per launch "
                         "(ratio to the rocprofv3 average %.3f); the profiler's own "
                         "per-dispatch work delays the events in the run above\n"
                         % (u[1], u[0] * 1e3, u[0] * 1e3 / avg_us))
        fh.write("- roofline: achieved %.3f %s of %.1f (frac %.4f)\n"
                 % (rf["achieved"], rf["unit"], rf["peak"], rf["frac"]))
        fh.write("- whole call: %.2f us, %.3f %s\n"
                 % (line["ms_per_step"] * 1e3, line["value"], line["unit"]))
    return out


def _counter(run_dir: str, counter: str):
    """Per-dispatch (dispatch id, kernel name, value) of one counter, with
    the values of all hardware instances of a dispatch summed."""
    with open(_csv(run_dir, "counter_collection.csv")) as fh:
        rows = list(csv.DictReader(fh))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = per.get(d, (r["Kernel_Name"], 0.0))
        per[d] = (name, v + float(r["Counter_Value"]))
    return [(d, per[d][0], per[d][1]) for d in sorted(per)]


def _counter_max(run_dir: str, counter: str):
    """Per-dispatch (dispatch id, kernel name, value) of one counter, the
    largest value over its hardware instances (for cycle counters that every
    instance counts in parallel)."""
    with open(_csv(run_dir, "counter_collection.csv")) as fh:
        rows = list(csv.DictReader(fh))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = per.get(d, (r["Kernel_Name"], 0.0))
        per[d] = (name, max(v, float(r["Counter_Value"])))
    return [(d, per[d][0], per[d][1]) for d in sorted(per)]


def _kernel_and_copy(run_dir: str, counter: str, short: str):
    disp = _counter(run_dir, counter)
    copies = disp[-CALIBRATION_COPIES:]
    if len(copies) < CALIBRATION_COPIES or not all("copy" in n.lower() for _, n, _ in copies):
        raise ValueError("the last %d dispatches in %s are not the calibration copies"
                         % (CALIBRATION_COPIES, run_dir))
    main = [(d, n, v) for d, n, v in disp if _matches(n, short)]
    if not main:
        raise ValueError("kernel %s not in %s" % (short, run_dir))
    kib = sum(v for _, _, v in main) / len(main)
    ckib = sum(v for _, _, v in copies) / len(copies)
    return main[0][1], len(main), kib, copies[0][1], ckib


def write_traffic(fetch_dir: str, write_dir: str, bench_log: str, workload: str,
                  copy_mib: int, command_fetch: str, command_write: str,
                  out_dir: str = PROFILES) -> str:
    line = _bench_line(bench_log)
    plan = line["config"]["plan"]
    variant, dtype = plan_variant(plan), line["dtype"]
    short = kernel_name(variant, dtype)
    kname, nf, fkib, cname, cfkib = _kernel_and_copy(fetch_dir, "FETCH_SIZE", short)
    _, nw, wkib, _, cwkib = _kernel_and_copy(write_dir, "WRITE_SIZE", short)
    copy_bytes = copy_mib * 1024 * 1024
    fscale = copy_bytes / (cfkib * 1024.0)
    wscale = copy_bytes / (cwkib * 1024.0)
    fbytes = fkib * 1024.0 * fscale
    wbytes = wkib * 1024.0 * wscale
    alg = line["roofline"].get("algorithmic_bytes")
    out = os.path.join(out_dir, "%s_%s_traffic.txt" % (short, workload))
    with open(out, "w") as fh:
        fh.write("# HBM traffic per launch of %s on %s (rocprofv3 --pmc, scaled by a\n"
                 "# plain device copy of %d MiB run at the end of the same program)\n"
                 % (short, workload, copy_mib))
        for k, v in [("kernel", short), ("workload", workload), ("plan", plan),
                     ("source_fingerprint", fingerprint(variant, dtype)),
                     ("command_fetch", command_fetch), ("command_write", command_write),
                     ("kernel_name", kname), ("fetch_dispatches", nf), ("write_dispatches", nw),
                     ("fetch_kib_per_dispatch", "%.3f" % fkib),
                     ("write_kib_per_dispatch", "%.3f" % wkib),
                     ("copy_kernel_name", cname), ("copy_bytes", copy_bytes),
                     ("copy_fetch_kib", "%.3f" % cfkib), ("copy_write_kib", "%.3f" % cwkib),
                     ("fetch_scale", "%.5f" % fscale), ("write_scale", "%.5f" % wscale),
                     ("fetch_bytes", "%.0f" % fbytes), ("write_bytes", "%.0f" % wbytes),
                     ("traffic_bytes", "%.0f" % (fbytes + wbytes)),
                     ("algorithmic_bytes", alg if alg is not None else "n/a")]:
            fh.write("%s: %s\n" % (k, v))
    return out


MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
SIMDS = 1024      # MI355X: 256 compute units x 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the 8 XCDs' own counters
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}


def write_mfma(run_dir: str, stats_dir: str, bench_log: str, workload: str, command: str,
               out_dir: str = PROFILES) -> str:
    """MFMA counters per launch of the main kernel, from a --pmc run of
    MFMA_COUNTERS; the launch duration is the kernel-trace average of the
    --stats run in stats_dir."""
    line = _bench_line(bench_log)
    plan = line["config"]["plan"]
    variant, dtype = plan_variant(plan), line["dtype"]
    short = kernel_name(variant, dtype)

    def per_launch(counter, reduce_max=False, optional=False):
        disp = (_counter_max if reduce_max else _counter)(run_dir, counter)
        if not disp and optional:
            return None, 0, 0.0
        main = [(d, n, v) for d, n, v in disp if _matches(n, short)]
        if not main:
            raise ValueError("kernel %s not in %s" % (short, run_dir))
        return main[0][1], len(main), sum(v for _, _, v in main) / len(main)

    kname, nd, mops32 = per_launch("SQ_INSTS_VALU_MFMA_MOPS_F32")
    _, _, mopsbf = per_launch("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    _, _, mopsh = per_launch("SQ_INSTS_VALU_MFMA_MOPS_F16", optional=True)
    mops16 = mopsbf + mopsh
    _, _, busy = per_launch("SQ_VALU_MFMA_BUSY_CYCLES")
    _, _, gui = per_launch("GRBM_GUI_ACTIVE", reduce_max=True)
    with open(_csv(stats_dir, "kernel_stats.csv")) as fh:
        st = [r for r in csv.DictReader(fh) if _matches(r["Name"], short)]
    if not st:
        raise ValueError("kernel %s not in %s" % (short, stats_dir))
    dur_s = float(st[0]["AverageNs"]) * 1e-9
    flops = (mops32 + mops16) * 512.0
    peak = PEAK_TFLOPS[dtype] * 1e12
    out = os.path.join(out_dir, "%s_%s_mfma.txt" % (short, workload))
    with open(out, "w") as fh:
        fh.write("# Matrix-core work per launch of %s on %s (rocprofv3 --pmc %s)\n"
                 "# counter_flops = (MOPS_F32 + MOPS_BF16 + MOPS_F16) * 512, padded lanes\n"
                 "# included;\n"
                 "# counter_util = counter_flops / (kernel-trace average duration * peak);\n"
                 "# busy_util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs * %d\n"
                 "# SIMDs), rocprofv3's MfmaUtil expression with the GUI-active cycles, which\n"
                 "# the counter reports summed over the XCDs, taken per XCD\n"
                 % (short, workload, " ".join(MFMA_COUNTERS), XCDS, SIMDS))
        for k, v in [("kernel", short), ("workload", workload), ("plan", plan),
                     ("source_fingerprint", fingerprint(variant, dtype)),
                     ("command", command), ("kernel_name", kname), ("dispatches", nd),
                     ("mops_f32_per_dispatch", "%.0f" % mops32),
                     ("mops_bf16_per_dispatch", "%.0f" % mopsbf),
                     ("mops_f16_per_dispatch", "%.0f" % mopsh),
                     ("mfma_busy_cycles_per_dispatch", "%.0f" % busy),
                     ("gui_active_cycles_per_dispatch", "%.0f" % gui),
                     ("kernel_trace_avg_us", "%.3f" % (dur_s * 1e6)),
                     ("peak_tflops", PEAK_TFLOPS[dtype]),
                     ("counter_flops", "%.0f" % flops),
                     ("counter_tflops", "%.3f" % (flops / dur_s / 1e12)),
                     ("counter_util", "%.4f" % (flops / dur_s / peak)),
                     ("busy_util", "%.4f" % (busy / (gui / XCDS * SIMDS) if gui else 0.0))]:
            fh.write("%s: %s\n" % (k, v))
    return out


def read_mfma(kernel: str, workload: str, plan: str, variant: str, dtype: str):
    """Counter-measured MFMA figures per launch from the committed summary, or
    None when there is none or the kernel's sources or plan changed since."""
    path = os.path.join(PROFILES, "%s_%s_mfma.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("plan") != plan or kv.get("source_fingerprint") != fingerprint(variant, dtype):
            return None
        return {"counter_flops": float(kv["counter_flops"]),
                "counter_util": float(kv["counter_util"]),
                "busy_util": float(kv["busy_util"])}
    except (KeyError, ValueError, FileNotFoundError):
        return None


def read_traffic(kernel: str, workload: str, plan: str, variant: str, dtype: str):
    """Scaled HBM bytes per launch from the committed traffic summary, or None
    when there is none or when the kernel's sources or plan changed since."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("plan") != plan or kv.get("source_fingerprint") != fingerprint(variant, dtype):
            return None
        return {"bytes": float(kv["traffic_bytes"]), "fetch_bytes": float(kv["fetch_bytes"]),
                "write_bytes": float(kv["write_bytes"])}
    except (KeyError, ValueError, FileNotFoundError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m conv2d_backward_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--run-dir", required=True)
    s.add_argument("--bench-log", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out-dir", default=PROFILES)
    s.add_argument("--plain-bench-log", default=None,
                   help="log of a bench.py run without the profiler, for comparison")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-dir", required=True)
    t.add_argument("--write-dir", required=True)
    t.add_argument("--bench-log", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out-dir", default=PROFILES)
    m = sub.add_parser("mfma")
    m.add_argument("--run-dir", required=True)
    m.add_argument("--stats-dir", required=True)
    m.add_argument("--bench-log", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--out-dir", default=PROFILES)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(write_stats(a.run_dir, a.bench_log, a.workload, a.command, a.out_dir,
                          plain_log=a.plain_bench_log))
    elif a.cmd == "mfma":
        print(write_mfma(a.run_dir, a.stats_dir, a.bench_log, a.workload, a.command, a.out_dir))
    else:
        print(write_traffic(a.fetch_dir, a.write_dir, a.bench_log, a.workload, a.copy_mib,
                            a.command_fetch, a.command_write, a.out_dir))


if __name__ == "__main__":
    main()
