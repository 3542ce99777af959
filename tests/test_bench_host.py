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


def test_default_headline_is_the_large_workload():
    args = bench.parse([])
    assert args.workload == bench.HEADLINE_WORKLOAD
    assert inputs.WORKLOADS[args.workload].name == "gemm_large_8192x8192x8192"
    assert args.gpus == 1 and not args.no_extras
    assert args.warmup == 10 and args.warmup_seconds > 0


def _fake_bench(index):
    """A Bench with its host-side fields set, as the GPU run would set them."""
    wl = inputs.WORKLOADS[index]
    _, shapes = inputs.workload_shapes(index)
    b = object.__new__(bench.Bench)
    b.wl, b.shapes, b.seed, b.copies = wl, shapes, 1000 + index, 3
    b.probs = [inputs.Problem(M, N, K, None, None, None, None) for (M, N, K) in shapes]
    b.flops = inputs.flops(shapes)
    b.alg_bytes = inputs.algorithmic_bytes(shapes)
    b.blocked = b.pow2 = b.device_table = False
    b.plan = lambda: {"kernel": 1}
    return b


def _fake_timing(kern_us):
    import numpy as np
    return {"wall_s": kern_us * 1e-6 * 20 * 1.05, "kern_s": kern_us * 1e-6,
            "each_us": np.full(20, kern_us), "host_us": 5.0, "warm_s": kern_us * 0.9e-6,
            "warmup_steps_run": 40}


def test_output_line_carries_every_field():
    """The JSON line of a run: the benchmark line's fields, the roofline and CPU
    baseline objects, the other workloads and the system metadata."""
    args = bench.parse(["--steps", "20", "--warmup", "5"])
    heads = {}
    extras = {}
    for i in range(len(inputs.WORKLOADS)):
        fb = _fake_bench(i)
        s = fb.summary(_fake_timing(900.0 if i == 2 else 30.0))
        if i == args.workload:
            heads = (fb, s)
        else:
            extras[fb.wl.name] = s
    fb, head = heads
    cpu = {"value": 0.04, "unit": "TFLOPS", "cores": 16, "kind": "oracle", "sample": "x",
           "affinity_cores": 16, "omp_num_threads": "16"}
    system = {"gpu": "x", "rocm": bench.rocm_version(), "torch_hip": None,
              "gfx_clock_under_headline_load": {"median_mhz": 1700.0},
              "affinity_cores": bench.affinity_cores(), "omp_num_threads": None}
    out = bench.compose(args, fb.wl, fb.seed, fb.copies, fb.flops, _fake_timing(900.0), head, extras,
                        cpu, system)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "warmup_steps_run", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "pct_fp4_peak", "pct_fp16_peak", "workloads", "system"):
        assert key in out, key
    assert out["config"]["workload"] == "gemm_large_8192x8192x8192"
    assert out["dtype"] == "f16" and out["n_gpus"] == 1 and out["vs_baseline"] is None
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - fb.flops / 900e-6 / 1e12 / 2500.0) < 1e-12
    assert set(out["workloads"]) == {w.name for w in inputs.WORKLOADS} - {"gemm_large_8192x8192x8192"}
    small = out["workloads"]["gemm_smallM_64x7168x16384"]
    assert small["roofline"]["bound"] == "hbm" and small["roofline"]["unit"] == "GB/s"
    for s in out["workloads"].values():
        for key in ("mean_launch_us", "kernel_tflops", "pct_fp16_peak", "pct_fp4_peak", "hbm_gbps",
                    "roofline", "plan"):
            assert key in s
        assert "frac" in s["roofline"] and "traffic" in s["roofline"]
    assert out["workloads"]["gemm_128x128x256"]["roofline"].get("note", "").startswith("latency")
    for key in ("gpu", "rocm", "gfx_clock_under_headline_load", "affinity_cores", "omp_num_threads"):
        assert key in out["system"]
    assert out["cpu_baseline"]["cores"] >= 1 and "affinity_cores" in out["cpu_baseline"]


def test_clock_sampler_reports_without_a_gpu():
    """Without a readable clock the sampler returns an error record instead
    of raising (the bench line still prints)."""
    if bench.read_sclk_mhz() is None:
        r = bench.sample_gfx_clock(lambda i: None, 0.01)
        assert r == {"error": "no readable pp_dpm_sclk"}


def test_sclk_parsing(tmp_path, monkeypatch):
    """The clock is the DPM entry marked with '*'."""
    import glob as glob_mod
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1698Mhz *\n2: 2400Mhz\n")
    monkeypatch.setattr(glob_mod, "glob", lambda pattern: [str(f)])
    assert bench.read_sclk_mhz() == 1698.0
    f.write_text("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz() == 94.0


def test_metadata_helpers():
    assert bench.affinity_cores() >= 1
    v = bench.rocm_version()
    assert v is None or v[0].isdigit()


def test_settle_warmup_runs_until_the_time_has_passed():
    """The untimed steps after --warmup double until --warmup-seconds of wall
    time have passed; with 0 seconds exactly --warmup steps run."""
    calls, syncs = [], []
    now = {"t": 0.0}

    def clock():
        return now["t"]

    def step(i):
        calls.append(i)
        now["t"] += 0.001  # one step takes a millisecond

    assert bench.settle_warmup(step, 10, 0.0, lambda: syncs.append(1), clock) == 10
    assert calls == list(range(10)) and len(syncs) == 1
    calls.clear()
    now["t"] = 0.0
    done = bench.settle_warmup(step, 10, 0.05, lambda: None, clock)
    assert calls == list(range(done))           # consecutive step indices
    assert done == 80                            # 10 -> 20 -> 40 -> 80 steps: 80 ms >= 50 ms
