"""Host logic of the rocprofv3 summaries (no GPU): counter parsing, the
copy-kernel scaling, and that bench.py's traffic figure is dropped once the
kernel's sources or plan no longer match the summary."""
import csv
import json
import os

import pytest

from conv2d_backward_amd import profiling

PLAN = "variant=halo dtype=f32 ws_bytes=1 launches=1 [tile=14x14]"
KNAME = "void gi::(anonymous namespace)::gi_halo_f32<13, 2, 512u, 1, 2>(gi::HaloArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, counter, rows):
    """rows: (kernel name, per-instance values) in dispatch order."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, (name, vals) in enumerate(rows, 1):
            for v in vals:
                w.writerow([d, name, counter, v])


def _bench_log(path, workload="resnet_stage_3x3"):
    line = {"dtype": "f32", "config": {"plan": PLAN, "workload": workload},
            "roofline": {"algorithmic_bytes": 1000, "kernel_ms": 0.08},
            "steps": 3, "warmup": 1}
    with open(path, "w") as fh:
        fh.write("noise\n" + json.dumps(line) + "\n")


def test_traffic_scaled_by_copy(tmp_path):
    mib = 4
    copy_b = mib * 1024 * 1024
    # The copy reads copy_b bytes but its FETCH counter says half (in KiB);
    # writes read exactly.  Values of several hardware instances add up.
    fetch_rows = [("other", [7.0]), (KNAME, [100.0, 100.0]), (KNAME, [300.0, 100.0])]
    fetch_rows += [(COPY, [copy_b / 2048 / 2, copy_b / 2048 / 2])] * 3
    write_rows = [(KNAME, [50.0]), (KNAME, [50.0])] + [(COPY, [copy_b / 1024])] * 3
    _counter_csv(str(tmp_path / "f"), "FETCH_SIZE", fetch_rows)
    _counter_csv(str(tmp_path / "w"), "WRITE_SIZE", write_rows)
    _bench_log(str(tmp_path / "b.log"))
    out = profiling.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"),
                                  str(tmp_path / "b.log"), "wl", mib, "cf", "cw",
                                  out_dir=str(tmp_path))
    kv = dict(ln.split(": ", 1) for ln in open(out).read().splitlines()
              if not ln.startswith("#"))
    assert float(kv["fetch_kib_per_dispatch"]) == pytest.approx(300.0)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0, rel=1e-4)
    assert float(kv["write_scale"]) == pytest.approx(1.0, rel=1e-4)
    assert float(kv["fetch_bytes"]) == pytest.approx(300 * 1024 * 2, rel=1e-4)
    assert float(kv["write_bytes"]) == pytest.approx(50 * 1024, rel=1e-4)
    assert kv["fetch_dispatches"] == "2"


def test_traffic_rejects_missing_copies(tmp_path):
    _counter_csv(str(tmp_path / "f"), "FETCH_SIZE", [(KNAME, [1.0])] * 4)
    _counter_csv(str(tmp_path / "w"), "WRITE_SIZE", [(KNAME, [1.0])] * 4)
    _bench_log(str(tmp_path / "b.log"))
    with pytest.raises(ValueError):
        profiling.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"),
                                str(tmp_path / "b.log"), "wl", 4, "a", "b",
                                out_dir=str(tmp_path))


def test_read_traffic_checks_plan_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path))
    fp = profiling.fingerprint("halo", "f32")
    path = tmp_path / "gi_halo_f32_wl_traffic.txt"
    path.write_text("# x\nplan: %s\nsource_fingerprint: %s\ntraffic_bytes: 123\n"
                    "fetch_bytes: 100\nwrite_bytes: 23\n" % (PLAN, fp))
    got = profiling.read_traffic("gi_halo_f32", "wl", PLAN, "halo", "f32")
    assert got == {"bytes": 123.0, "fetch_bytes": 100.0, "write_bytes": 23.0}
    # Another plan, or sources that changed since: no figure.
    assert profiling.read_traffic("gi_halo_f32", "wl", PLAN + " ", "halo", "f32") is None
    path.write_text(path.read_text().replace(fp, "0" * 16))
    assert profiling.read_traffic("gi_halo_f32", "wl", PLAN, "halo", "f32") is None
    assert profiling.read_traffic("gi_halo_f32", "none", PLAN, "halo", "f32") is None


def test_fingerprint_covers_every_kernel():
    seen = {profiling.fingerprint(v, d) for v, d in profiling.KERNEL_SOURCES}
    # generic f32 and bf16 share one source file, so do gw and gwd, and the
    # 16-bit halo and image kernels' bf16 and fp16 instantiations
    assert len(seen) == 8


def test_mfma_summary(tmp_path, monkeypatch):
    """Counter flops and utilisation per launch: instance values add up for
    the instruction and busy counters, the GUI-active cycles take the largest
    instance (per XCD after dividing the reported sum by the XCD count), and
    the duration comes from the kernel-trace statistics."""
    os.makedirs(str(tmp_path / "m"))
    with open(str(tmp_path / "m" / "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d in (1, 2):
            for v in (600.0, 400.0):
                w.writerow([d, KNAME, "SQ_INSTS_VALU_MFMA_MOPS_F32", v])
            w.writerow([d, KNAME, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0])
            for v in (512.0, 512.0):
                w.writerow([d, KNAME, "SQ_VALU_MFMA_BUSY_CYCLES", v])
            for v in (1.0, 2.0):
                w.writerow([d, KNAME, "GRBM_GUI_ACTIVE", v])
        w.writerow([3, "other", "SQ_INSTS_VALU_MFMA_MOPS_F32", 9e9])
    os.makedirs(str(tmp_path / "s"))
    with open(str(tmp_path / "s" / "run_kernel_stats.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([KNAME, 10, 100, 10, 100])
    _bench_log(str(tmp_path / "b.log"))
    out = profiling.write_mfma(str(tmp_path / "m"), str(tmp_path / "s"),
                               str(tmp_path / "b.log"), "wl", "cmd", out_dir=str(tmp_path))
    kv = dict(ln.split(": ", 1) for ln in open(out).read().splitlines()
              if not ln.startswith("#"))
    assert float(kv["counter_flops"]) == 1000 * 512
    # 512000 flops in 10 ns against 157.3 TFLOP/s.
    assert float(kv["counter_util"]) == pytest.approx(512000 / 1e-8 / 157.3e12, rel=1e-3)
    assert float(kv["busy_util"]) == pytest.approx(1024 / (2 / profiling.XCDS * profiling.SIMDS),
                                                   rel=1e-6)
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path))
    assert profiling.read_mfma("gi_halo_f32", "wl", PLAN, "halo", "f32")["counter_flops"] == 512000
    assert profiling.read_mfma("gi_halo_f32", "wl", PLAN + "x", "halo", "f32") is None


def test_plan_variant_and_kernel_names():
    """Plans map to the kernel that runs them: the 16-bit whole-image plan to
    gi_img16 (its bf16 and fp16 instantiations), the column plan to
    gi_col2im_f32."""
    img = ("variant=halo dtype=bf16 ws_bytes=4718592 launches=2 [image kernel cfg=0 nb=13 "
           "wgs=64x4 lds=109568 halo=16x16 pitch=30 chunks=16]")
    assert profiling.plan_variant(img) == "img16"
    assert profiling.kernel_name("img16", "bf16") == "gi_img16_bf16"
    bf = "void gi::(anonymous namespace)::gi_img16<false, 13, 9, 3, 30, 16>(gi::Img16Args)"
    hf = "void gi::(anonymous namespace)::gi_img16<true, 13, 9, 3, 30, 16>(gi::Img16Args)"
    assert profiling._matches(bf, "gi_img16_bf16") and not profiling._matches(hf, "gi_img16_bf16")
    assert profiling._matches(hf, "gi_img16_f16") and not profiling._matches(bf, "gi_img16_f16")
    col = "variant=col2im dtype=f32 ws_bytes=0 launches=1 [tile=56x56 wgs=256 cols=147]"
    assert profiling.plan_variant(col) == "col2im"
    assert profiling._matches("void gi::(anonymous namespace)::gi_col2im_f32<10, 2, 64>"
                              "(gi::Col2imArgs)", profiling.kernel_name("col2im", "f32"))
    assert profiling.plan_variant("variant=halo dtype=f32 ws_bytes=1 launches=1 [nb=13]") == "halo"
