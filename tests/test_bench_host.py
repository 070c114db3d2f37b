"""Host-side logic of the benchmark (no GPU): the kernel-source hash that
gates recorded HBM counter readings, the scaling of FETCH_SIZE / WRITE_SIZE
readings by the plain-copy calibration, and the one-GPU rule."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _point_sources_at(monkeypatch, tmp_path, texts):
    names = []
    for i, t in enumerate(texts):
        p = tmp_path / f"k{i}.h"
        p.write_text(t)
        names.append(p.name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", names)


def test_source_hash_ignores_comments_and_spacing(monkeypatch, tmp_path):
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n/* block\n comment */\nint g;\n"
    _point_sources_at(monkeypatch, tmp_path, [code])
    h0 = bench.kernel_source_hash()
    _point_sources_at(monkeypatch, tmp_path, [
        "// header comment\nint   f(int a)\n{\n\n  return a + 1;  // a different comment\n}\nint g;   /* x */\n"])
    assert bench.kernel_source_hash() == h0
    _point_sources_at(monkeypatch, tmp_path, [code.replace("a + 1", "a + 2")])
    assert bench.kernel_source_hash() != h0


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy(monkeypatch, tmp_path):
    """The copy kernel moves exactly 256 MiB each way: a FETCH_SIZE reading of
    half that gives a read factor of 2, a full WRITE_SIZE reading a write
    factor of 1; the decode kernel's readings (mean over dispatches) are scaled
    by them.  The largest copy dispatch is the calibration one."""
    kib = bench.COPY_BYTES / 1024
    head = "void iq::(anonymous namespace)::" + bench.TRAFFIC_KERNELS["headline"] + "(iq::DecodeArgs)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 12.0), ("__amd_rocclr_copyBuffer", kib / 2),
                                       (head, 1000.0), (head, 1200.0), ("other_kernel", 5.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 3.0), ("__amd_rocclr_copyBuffer", kib),
                                       (head, 40.0), (head, 60.0)])
    out_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out_file))
    assert bench.summarize_counters(str(fetch), str(write)) == 0
    rec = json.loads(out_file.read_text())
    assert rec["copy_calibration"]["read_factor"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    entry = rec["workloads"]["headline"]
    assert entry["dispatches"] == 2
    assert entry["hbm_bytes_per_launch"] == int(round((1100.0 * 2.0 + 50.0 * 1.0) * 1024))
    assert "batched_append_c5" not in rec["workloads"]          # no dispatches of that kernel
    # reported while the sources are those the readings were taken on
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.recorded_traffic("headline") == entry["hbm_bytes_per_launch"]
    rec["kernel_source_hash"] = "0" * 16
    out_file.write_text(json.dumps(rec))
    assert bench.recorded_traffic("headline") is None


def test_counter_summary_needs_the_copy(monkeypatch, tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("partial_kernel", 1.0)])
    _counter_csv(write, "WRITE_SIZE", [("partial_kernel", 1.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(fetch), str(write))


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
