"""Host logic of bench.py (no GPU): the roofline record of the dominant kernel
and the validity rules of the committed HBM-traffic records."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _stat(name, launches, total_ms, flops=0.0, nbytes=0.0):
    return {"name": name, "launches": launches, "total_ms": total_ms, "flops": flops, "bytes": nbytes}


def test_roofline_picks_the_largest_summed_time_and_prices_flops():
    stats = [_stat("fwd_gemm", 4, 28.0, flops=4 * 9.5e12), _stat("dw_gemm", 2, 30.0, flops=2 * 19e12),
             _stat("lse_kl", 4, 0.2, nbytes=4 * 5.8e7)]
    r = bench.roofline_of(stats, lambda k: 123 if k == "dw_gemm" else None)
    assert r["kernel"] == "dw_gemm" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["avg_launch_ms"] == 15.0
    assert r["achieved"] == pytest.approx(19e12 / 15e-3 / 1e12, rel=1e-4)
    assert r["peak"] == bench.BF16_PEAK_TFLOPS
    assert r["frac"] == pytest.approx(r["achieved"] / bench.BF16_PEAK_TFLOPS, abs=1e-4)
    assert r["traffic"] == 123
    r32 = bench.roofline_of(stats, lambda k: None, bench.FP32_MFMA_PEAK_TFLOPS)
    assert r32["peak"] == bench.FP32_MFMA_PEAK_TFLOPS and r32["traffic"] is None


def test_roofline_of_a_memory_bound_dominant_kernel():
    r = bench.roofline_of([_stat("dh_reduce", 4, 2.0, nbytes=4 * 2.0e9)], lambda k: None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(2.0e9 / 0.5e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS, abs=1e-4)


def test_committed_traffic_records_are_used_only_for_their_source_and_workload():
    # every committed record names its kernel, workload, the kernel source and the host
    # code (rows per launch) it was taken on; it is reported only while both are
    # unchanged, and only for that workload
    for k in ("fwd_gemm", "recompute_gemm", "dh_gemm", "dw_gemm"):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"traffic_{k}.json")))
        assert rec["kernel"] == k and rec["hbm_bytes_per_launch"] > 0
        same = True
        for f, h in ((rec["source_file"], rec["source_sha256"]), (rec["driver_file"], rec["driver_sha256"])):
            src = open(os.path.join(ROOT, "chunked_sparse_kl_amd", "csrc", f), "rb").read()
            same = same and hashlib.sha256(src).hexdigest() == h
        assert bench.kernel_traffic(k, rec["workload"]) == (rec["hbm_bytes_per_launch"] if same else None)
        assert bench.kernel_traffic(k, "another workload chunk 64") is None


def test_traffic_record_of_another_source_is_ignored(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    csrc = tmp_path / "chunked_sparse_kl_amd" / "csrc"
    prof.mkdir()
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// current source\n")
    rec = {"kernel": "x_gemm", "workload": "w chunk 8", "source_file": "k.hip",
           "source_sha256": hashlib.sha256(b"// older source\n").hexdigest(), "hbm_bytes_per_launch": 5}
    (prof / "traffic_x_gemm.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_traffic("x_gemm", "w chunk 8") is None
    rec["source_sha256"] = hashlib.sha256(b"// current source\n").hexdigest()
    (prof / "traffic_x_gemm.json").write_text(json.dumps(rec))
    assert bench.kernel_traffic("x_gemm", "w chunk 8") == 5
    assert bench.kernel_traffic("missing_gemm", "w chunk 8") is None
    # a record that also names the host code choosing the rows per launch
    (csrc / "api.cpp").write_text("// launches per pair of chunks\n")
    rec["driver_file"] = "api.cpp"
    rec["driver_sha256"] = hashlib.sha256(b"// launches per chunk\n").hexdigest()
    (prof / "traffic_x_gemm.json").write_text(json.dumps(rec))
    assert bench.kernel_traffic("x_gemm", "w chunk 8") is None
    rec["driver_sha256"] = hashlib.sha256(b"// launches per pair of chunks\n").hexdigest()
    (prof / "traffic_x_gemm.json").write_text(json.dumps(rec))
    assert bench.kernel_traffic("x_gemm", "w chunk 8") == 5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_runs_on_the_granted_host_threads(monkeypatch):
    import numpy as np
    cpus = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert bench.host_cpus() == (cpus, min(cpus, 2))
    _, _, used, seen = bench.timed_oracle(lambda: np.ones((64, 64)) @ np.ones((64, 64)))
    assert used == min(cpus, 2) and seen == cpus
    monkeypatch.delenv("OMP_NUM_THREADS")
    _, _, used, _ = bench.timed_oracle(lambda: None)
    assert used == cpus
