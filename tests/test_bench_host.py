"""Host-side logic of bench.py that needs no GPU: the single-GPU refusal,
and the HBM-traffic summary that fills the bench line's roofline.traffic
(counter values in KiB per dispatch, scaled by a plain copy's reading)."""

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
        dict(Dispatch_Id=5, Kernel_Name="void moe::combine_kernel<float>(int)", Grid_Size=64,
             Counter_Name="FETCH_SIZE", Counter_Value=9e9)])
    w = _counters(tmp_path / "w", [
        dict(Dispatch_Id=3, Kernel_Name=k13, Grid_Size=256, Counter_Name="WRITE_SIZE",
             Counter_Value=10.0),
        dict(Dispatch_Id=7, Kernel_Name=k13, Grid_Size=256, Counter_Name="WRITE_SIZE",
             Counter_Value=30.0)])
    path = bench.summarize_traffic("skew", [f, w, cf, cw], "cmd")
    t = json.load(open(path))
    assert t["calibration"]["FETCH_SIZE_bytes_per_counted_byte"] == 2.0
    assert t["calibration"]["WRITE_SIZE_bytes_per_counted_byte"] == 1.0
    assert [r["fetch_bytes"] for r in t["launches"]] == [2 * 1000 * 1024, 2 * 3000 * 1024]
    assert [r["write_bytes"] for r in t["launches"]] == [10 * 1024, 30 * 1024]
    assert t["traffic_bytes_per_launch"] == (2 * 4000 * 1024 + 40 * 1024) // 2
    # read back only while the sources are the ones the counters were taken on
    assert bench.load_traffic("skew") == t["traffic_bytes_per_launch"]
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
