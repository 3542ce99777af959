"""Host-side logic of bench.py, on the CPU (no GPU call)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from grouped_gemm_nvfp4_amd import inputs  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    table = tmp_path / "traffic.txt"
    table.write_text("# comment\nwl_a %s 123\nwl_b %s 456\n" % (sha, "0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.measured_traffic("wl_a") == 123.0
    assert bench.measured_traffic("wl_b") is None      # taken on another source
    assert bench.measured_traffic("wl_c") is None      # never measured


def test_cpu_baseline_reports_the_oracle():
    probs = inputs.draw_problems(7, [(48, 64, 256)])
    cpu = bench.cpu_baseline(probs, 0.05)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOPS"
    assert cpu["value"] > 0 and cpu["cores"] >= 1
    assert "workload" in cpu["sample"] or "rows" in cpu["sample"]
    assert "cpu_model" in cpu and "omp_num_threads" in cpu


def test_shape_option_parsing():
    assert bench.parse_shape("64,4096,7168") == (64, 4096, 7168)
    for bad in ("64,4096", "64,4096,70", "0,8,32", "a,b,c"):
        with pytest.raises(SystemExit):
            bench.parse_shape(bad)
