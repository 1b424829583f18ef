"""bench.py's host logic, on the CPU: the one-GPU refusal, the HBM-traffic
summary of two rocprofv3 counter runs (each counter scaled by what it reads
for a calibration kernel of known size), and the rule that committed
counters count only while they were taken on the current kernel sources."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CAL_NAME = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctor_add<float>, std::array<char*, 3ul> >"
ROW_NAME = "void nucleus::row_kernel<0, false, false>(nucleus::Params, nucleus::RowWork)"
OTHER_NAME = "void at::native::reduce_kernel<512, 1>(float*)"


def _counter_dir(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": "X", "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_pmc_summary_scales_each_counter_by_the_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    # The calibration kernel reads and writes CAL_BYTES: FETCH_SIZE reports
    # half of them (factor 2), WRITE_SIZE all of them (factor 1).
    cal_fetch = bench.CAL_BYTES / 2 / 1024
    cal_write = bench.CAL_BYTES / 1024
    _counter_dir(tmp_path / "fetch", [(CAL_NAME, cal_fetch), (ROW_NAME, 1000.0), (ROW_NAME, 1200.0),
                                      (OTHER_NAME, 5.0)])
    _counter_dir(tmp_path / "write", [(CAL_NAME, cal_write), (ROW_NAME, 16.0), (ROW_NAME, 16.0)])
    B, V = 4, 1000
    out = bench.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), "tiny", (B, V), "f32")
    assert out["fetch"]["scale_factor"] == pytest.approx(2.0)
    assert out["write"]["scale_factor"] == pytest.approx(1.0)
    fk = out["fetch"]["kernels"]
    assert set(fk) == {"row_kernel"}  # torch's own kernels are not the sampler's
    assert fk["row_kernel"]["dispatches"] == 2
    fetch = 1100.0 * 1024 * 2.0
    write = 16.0 * 1024 * 1.0
    assert fk["row_kernel"]["bytes_per_dispatch"] == pytest.approx(fetch)
    assert out["traffic_bytes_per_launch"] == pytest.approx(fetch + write)
    assert out["algorithmic_bytes_per_launch"] == B * V * 4
    assert out["fetch_over_algorithmic"] == pytest.approx(fetch / (B * V * 4))
    with open(tmp_path / "profiles" / "pmc_tiny.json") as f:
        assert json.load(f)["traffic_bytes_per_launch"] == pytest.approx(fetch + write)


def test_pmc_summary_needs_a_calibration_dispatch(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _counter_dir(tmp_path / "fetch", [(ROW_NAME, 1000.0)])
    _counter_dir(tmp_path / "write", [(ROW_NAME, 16.0)])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), "tiny", (4, 1000), "f32")


def test_traffic_counts_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    path = tmp_path / "profiles" / "pmc_tiny.json"
    path.write_text(json.dumps({"kernel_hash": bench.kernel_hash(), "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_from_profile("tiny", 100.0) == 123.0
    path.write_text(json.dumps({"kernel_hash": "0" * 16, "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_from_profile("tiny", 100.0) is None
    assert bench.traffic_from_profile("absent", 100.0) is None


def test_kernel_hash_covers_every_library_source():
    csrc = os.path.join(ROOT, "nucleus_sampling_amd", "csrc")
    want = sorted(os.path.relpath(os.path.join(csrc, n), ROOT) for n in os.listdir(csrc) if n.endswith((".h", ".hip")))
    assert bench.KERNEL_SOURCES == want
    assert len(want) >= 10
