"""Host logic of bench.py (no GPU): the one-GPU contract and the counter summary."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_counters(d, sub, rows):
    os.makedirs(os.path.join(d, sub), exist_ok=True)
    with open(os.path.join(d, sub, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_copy(tmp_path):
    import bench
    d = str(tmp_path)
    n_copy_kib = (256 << 20) / 1024.0
    # the copy reads half its bytes on FETCH_SIZE and all on WRITE_SIZE
    _write_counters(d, "FETCH_SIZE_copy", [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer",
                                                 Counter_Name="FETCH_SIZE", Counter_Value=n_copy_kib / 2)])
    _write_counters(d, "WRITE_SIZE_copy", [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer",
                                                 Counter_Name="WRITE_SIZE", Counter_Value=n_copy_kib)])
    # two dispatches of a kernel, each counter split over two rows (two XCD instances)
    rows_f = [dict(Dispatch_Id=i, Kernel_Name="void moe::gate_up_mfma<2, 1, 1, 2, true>(moe::FfnArgs, int, int)",
                   Counter_Name="FETCH_SIZE", Counter_Value=v) for i in (5, 6) for v in (300.0, 200.0)]
    rows_w = [dict(Dispatch_Id=i, Kernel_Name="void moe::gate_up_mfma<2, 1, 1, 2, true>(moe::FfnArgs, int, int)",
                   Counter_Name="WRITE_SIZE", Counter_Value=v) for i in (5, 6) for v in (10.0, 6.0)]
    _write_counters(d, "FETCH_SIZE", rows_f)
    _write_counters(d, "WRITE_SIZE", rows_w)
    s = bench.summarize_counters(d)
    k = s["kernels"]["gate_up_mfma"]
    assert k["dispatches"] == 2
    assert abs(s["copy_calibration"]["fetch_factor"] - 2.0) < 1e-6
    assert abs(s["copy_calibration"]["write_factor"] - 1.0) < 1e-6
    # per dispatch: 500 KiB fetched (x2) and 16 KiB written
    assert k["fetch_bytes"] == 500 * 1024 * 2
    assert k["write_bytes"] == 16 * 1024
    assert k["hbm_bytes_per_launch"] == 500 * 1024 * 2 + 16 * 1024
    assert s["ffn_source_sha256"] == bench.ffn_source_hash()
    json.dumps(s)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    import bench
    a = tmp_path / "a.hip"
    a.write_text("int f() { return 1; }  // one\n/* block\ncomment */\n")
    monkeypatch.setattr(bench, "FFN_SOURCES", [str(a)])
    h1 = bench.ffn_source_hash()
    a.write_text("int f() {\n  return 1;   // another comment\n}\n")
    assert bench.ffn_source_hash() == h1
    a.write_text("int f() { return 2; }\n")
    assert bench.ffn_source_hash() != h1
