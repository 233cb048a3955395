"""Host-side logic of bench.py that needs no GPU: the single-GPU refusal,
the HBM-traffic summary that fills the bench line's roofline.traffic
(counter values in KiB per dispatch, scaled by a plain copy's reading), and
the matrix-core counter summary."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    return str(path)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda exclude=(): "cafe")
    os.makedirs(tmp_path / "profiles")
    k13 = "void moe::ffn13_gemm_kernel<unsigned short, 128, 2, 1, 4, true>(int)"
    k2 = "void moe::ffn2_gemm_kernel<unsigned short, 128, 2, 1, 4>(int)"
    cal = bench.COPY_CAL_BYTES
    # the copy of `cal` bytes reads cal/2 KiB-units on FETCH_SIZE (factor 2)
    # and cal on WRITE_SIZE (factor 1); other kernels are ignored
    cf = _counters(tmp_path / "cf", [
        dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=1,
             Counter_Name="FETCH_SIZE", Counter_Value=cal / 2 / 1024)])
    cw = _counters(tmp_path / "cw", [
        dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=1,
             Counter_Name="WRITE_SIZE", Counter_Value=cal / 1024)])
    f = _counters(tmp_path / "f", [
        dict(Dispatch_Id=3, Kernel_Name=k13, Grid_Size=256, Counter_Name="FETCH_SIZE",
             Counter_Value=1000.0),
        dict(Dispatch_Id=7, Kernel_Name=k13, Grid_Size=256, Counter_Name="FETCH_SIZE",
             Counter_Value=3000.0),
        dict(Dispatch_Id=4, Kernel_Name=k2, Grid_Size=128, Counter_Name="FETCH_SIZE",
             Counter_Value=500.0),
        dict(Dispatch_Id=5, Kernel_Name="void moe::combine_kernel<float>(int)", Grid_Size=64,
             Counter_Name="FETCH_SIZE", Counter_Value=9e9)])
    w = _counters(tmp_path / "w", [
        dict(Dispatch_Id=3, Kernel_Name=k13, Grid_Size=256, Counter_Name="WRITE_SIZE",
             Counter_Value=10.0),
        dict(Dispatch_Id=4, Kernel_Name=k2, Grid_Size=128, Counter_Name="WRITE_SIZE",
             Counter_Value=64.0),
        dict(Dispatch_Id=7, Kernel_Name=k13, Grid_Size=256, Counter_Name="WRITE_SIZE",
             Counter_Value=30.0)])
    path = bench.summarize_traffic("skew", [f, w, cf, cw], "the command")
    t = json.load(open(path))
    assert t["command"] == "the command"
    assert t["calibration"]["FETCH_SIZE_bytes_per_counted_byte"] == 2.0
    assert t["calibration"]["WRITE_SIZE_bytes_per_counted_byte"] == 1.0
    t13, t2 = t["ffn13"], t["ffn2"]
    assert [r["fetch_bytes"] for r in t13["launches"]] == [2 * 1000 * 1024, 2 * 3000 * 1024]
    assert [r["write_bytes"] for r in t13["launches"]] == [10 * 1024, 30 * 1024]
    assert t13["traffic_bytes_per_launch"] == (2 * 4000 * 1024 + 40 * 1024) // 2
    assert t2["traffic_bytes_per_launch"] == 2 * 500 * 1024 + 64 * 1024
    # read back only while the sources are the ones the counters were taken on
    assert bench.load_traffic("skew") == {"ffn13": t13["traffic_bytes_per_launch"],
                                          "ffn2": t2["traffic_bytes_per_launch"]}
    monkeypatch.setattr(bench, "kernel_source_sha", lambda exclude=(): "beef")
    assert bench.load_traffic("skew") is None


def test_traffic_summary_rejects_mismatched_runs(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda exclude=(): "cafe")
    os.makedirs(tmp_path / "profiles")
    k13 = "void moe::ffn13_gemm_kernel<unsigned short, 128, 2, 1, 4, true>(int)"
    cal = bench.COPY_CAL_BYTES
    cf = _counters(tmp_path / "cf", [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer",
                                          Grid_Size=1, Counter_Name="FETCH_SIZE",
                                          Counter_Value=cal / 1024)])
    cw = _counters(tmp_path / "cw", [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer",
                                          Grid_Size=1, Counter_Name="WRITE_SIZE",
                                          Counter_Value=cal / 1024)])
    f = _counters(tmp_path / "f", [dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=256,
                                        Counter_Name="FETCH_SIZE", Counter_Value=1.0)] * 2)
    w = _counters(tmp_path / "w", [dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=256,
                                        Counter_Name="WRITE_SIZE", Counter_Value=1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic("skew", [f, w, cf, cw], "cmd")


def test_matrix_core_summary(tmp_path, monkeypatch):
    """Counted flops (512 per MOPS unit) over the stats run's average
    duration, and MFMA busy cycles over 4 SIMDs x 256 CUs x one XCD's active
    cycles (GRBM_GUI_ACTIVE summed over 8 XCDs)."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda exclude=(): "cafe")
    os.makedirs(tmp_path / "profiles")
    k13 = "void moe::ffn13_big_kernel<unsigned short>(int)"
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e9, "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0,
            "SQ_INSTS_VALU_MFMA_MOPS_F6F4": 0.0, "SQ_VALU_MFMA_BUSY_CYCLES": 4 * 256 * 1000.0 * 0.5,
            "SQ_INSTS_MFMA": 1e6, "SQ_BUSY_CYCLES": 1.0, "GRBM_GUI_ACTIVE": 8 * 1000.0}
    pm = _counters(tmp_path / "pm", [dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1,
                                          Counter_Name=c, Counter_Value=v)
                                     for c, v in vals.items()])
    st = tmp_path / "st"
    os.makedirs(st)
    with open(st / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow(dict(Name=k13, Calls=2, TotalDurationNs=2 * 1024e3, AverageNs=1024e3,
                        MinNs=1024e3, MaxNs=1024e3))
    path = bench.summarize_pmc("prefill_bf16", [pm, str(st)], "cmd one ;; cmd two")
    text = open(path).read()
    assert "    cmd one" in text and "    cmd two" in text
    row = next(l for l in text.splitlines() if l.startswith("| ffn13 |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    flops = 512 * 2e9
    assert float(cells[-6]) == pytest.approx(flops / 1e12, rel=1e-3)
    assert float(cells[-5]) == pytest.approx(1024.0)
    assert float(cells[-4]) == pytest.approx(flops / 1024e-6 / 1e12, rel=1e-3)
    assert float(cells[-2]) == pytest.approx(50.0)


def test_memory_path_summary(tmp_path, monkeypatch):
    """Unit busy fractions per CU and XCD-cycle (each counter paired with its
    own pass's GRBM_GUI_ACTIVE) and the L2 hit rate, averaged per kind."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda exclude=(): "cafe")
    os.makedirs(tmp_path / "profiles")
    k13 = "void moe::ffn13_wide_kernel<unsigned char>(int)"
    k2 = "void moe::ffn2_wide_kernel<unsigned char>(int)"
    g = 8 * 1000.0  # one XCD active 1000 cycles
    a = _counters(tmp_path / "a", [
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="TA_TA_BUSY_sum",
             Counter_Value=256 * 800.0),
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="TD_TD_BUSY_sum",
             Counter_Value=256 * 900.0),
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="GRBM_GUI_ACTIVE",
             Counter_Value=g),
        dict(Dispatch_Id=2, Kernel_Name=k13, Grid_Size=1, Counter_Name="TA_TA_BUSY_sum",
             Counter_Value=256 * 300.0),
        dict(Dispatch_Id=2, Kernel_Name=k13, Grid_Size=1, Counter_Name="TD_TD_BUSY_sum",
             Counter_Value=256 * 700.0),
        dict(Dispatch_Id=2, Kernel_Name=k13, Grid_Size=1, Counter_Name="GRBM_GUI_ACTIVE",
             Counter_Value=g / 2),
        dict(Dispatch_Id=3, Kernel_Name=k2, Grid_Size=1, Counter_Name="TA_TA_BUSY_sum",
             Counter_Value=256 * 500.0),
        dict(Dispatch_Id=3, Kernel_Name=k2, Grid_Size=1, Counter_Name="GRBM_GUI_ACTIVE",
             Counter_Value=g)])
    b = _counters(tmp_path / "b", [
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="TCC_HIT_sum",
             Counter_Value=30.0),
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="TCC_MISS_sum",
             Counter_Value=70.0),
        dict(Dispatch_Id=1, Kernel_Name=k13, Grid_Size=1, Counter_Name="GRBM_GUI_ACTIVE",
             Counter_Value=g)])
    path = bench.summarize_mempath("fp8", [a, b], "cmd one ;; cmd two")
    text = open(path).read()
    assert "    cmd one" in text and "    cmd two" in text and "`cafe`" in text
    row13 = [c.strip() for c in next(l for l in text.splitlines() if l.startswith("| ffn13 |")).strip("|").split("|")]
    # TA: (0.8 + 0.6) / 2; TD: (0.9 + 1.4) / 2; no stall counters; L2 30 / 100
    assert row13[2:] == ["0.700", "1.150", "-", "-", "0.300"]
    row2 = [c.strip() for c in next(l for l in text.splitlines() if l.startswith("| ffn2 |")).strip("|").split("|")]
    assert row2[2] == "0.500" and row2[-1] == "-"
