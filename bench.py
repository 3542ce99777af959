#!/usr/bin/env python3
"""Throughput of the NVFP4 GEMM / grouped GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]

One step is one call of the library (nvfp4_gemm for a single product,
nvfp4_group_gemm for a grouped one) over one set of synthetic operands that
already sit in device memory.  The headline workload is the large
compute-bound product M = N = K = 8192; ``--workload`` picks another of the
named workloads in grouped_gemm_nvfp4_amd/inputs.py and ``--shape M,N,K`` any
single GEMM.  Unless ``--no-extras`` is given, every other named workload is
timed in the same run, the same way, and reported under ``"workloads"``.

Steps cycle over several identical copies of the operands whose total size
exceeds the 256 MiB Infinity Cache plus the L2s, so each step reads its
operands from HBM rather than from a cache warmed by the previous step.

Prints one JSON line: TFLOPS = sum 2*M*N*K / time, the roofline of the kernel
(algorithmic bytes or flops per launch over its mean launch duration: the
timed region measured with HIP events on the launch stream, divided by the
number of steps), and the CPU oracle's throughput on a bounded sample of the
headline workload.  The roofline's "traffic" (HBM bytes per launch from the
FETCH_SIZE and WRITE_SIZE counters) comes from profiles/hbm_traffic.txt and is
reported only while the kernel sources it was measured on are unchanged.  The
GPU's graphics clock (the driver's DPM table in sysfs) is sampled while the
headline workload runs back to back.

    python bench.py --copy-probe BYTES

runs a plain device-to-device copy of BYTES bytes a few times and exits: under
rocprofv3 --pmc it calibrates the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from grouped_gemm_nvfp4_amd import inputs  # noqa: E402

# MI355X published dense peaks
PEAK_HBM_GBPS = 8000.0
PEAK_FP16_TFLOPS = 2500.0
PEAK_FP4_TFLOPS = 10100.0
CACHE_BYTES = 256 * 2 ** 20 + 8 * 4 * 2 ** 20  # Infinity Cache + 8 XCD L2s

METRIC = "TFLOPS (2MNK/t) NVFP4 GEMM & grouped GEMM; % FP4 MFMA peak; HBM GB/s"
HEADLINE_WORKLOAD = 2  # gemm_large_8192x8192x8192

SHAPE_SEED = 2000  # inputs of a --shape run


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.25,
                    help="after the --warmup steps, keep stepping (untimed) until this much wall "
                         "time has passed, so that the timed steps run at the clock the sustained "
                         "load settles at (0: exactly --warmup steps)")
    ap.add_argument("--workload", type=int, default=HEADLINE_WORKLOAD,
                    help="index into grouped_gemm_nvfp4_amd.inputs.WORKLOADS (default %d, the "
                         "8192^3 product)" % HEADLINE_WORKLOAD)
    ap.add_argument("--shape", default=None, metavar="M,N,K",
                    help="time one GEMM of these sizes (seeded inputs, seed %d) instead of a "
                         "named workload" % SHAPE_SEED)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--copies", type=int, default=0,
                    help="operand copies to cycle over (0: enough to exceed the caches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0: skip)")
    ap.add_argument("--clock-seconds", type=float, default=0.5,
                    help="seconds of back-to-back headline steps during which the GPU clock is "
                         "sampled (0: skip)")
    ap.add_argument("--scale-layout", choices=("plain", "blocked"), default="plain",
                    help="scales as [rows][K/16] (default) or in the pages' blocked 512-byte atoms "
                         "(nvfp4_gemm_blocked / nvfp4_group_gemm_blocked)")
    ap.add_argument("--scales", choices=("general", "pow2"), default="general",
                    help="scales uniform over the 49 e4m3 codes in [0.125, 8] (default), or over their "
                         "seven powers of two, run on the FP4-MFMA path (nvfp4_gemm_pow2scale / "
                         "nvfp4_group_gemm_pow2scale)")
    ap.add_argument("--table", choices=("host", "device"), default="host",
                    help="grouped workloads: the problem table passed by value (default) or read on "
                         "the device (nvfp4_group_gemm_device: plan kernel + one-wave tiles)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    return ap.parse_args(argv)


KERNEL_DIR = os.path.join(ROOT, "grouped_gemm_nvfp4_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def parse_shape(text):
    """'M,N,K' -> (M, N, K): positive sizes, K a multiple of 32."""
    try:
        M, N, K = (int(x) for x in text.split(","))
    except ValueError:
        raise SystemExit("--shape takes M,N,K (three integers), got %r" % text)
    if min(M, N, K) < 1 or K % 32 != 0:
        raise SystemExit("--shape needs M, N, K >= 1 and K a multiple of 32, got %r" % text)
    return M, N, K


def kernel_source_sha():
    """sha256 over the device sources (csrc/*.hip and csrc/*.h, by name):
    what the traffic figures are keyed to."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode() + b"\0")
            with open(os.path.join(KERNEL_DIR, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch recorded for this workload, if they were measured
    on the current kernel sources (lines: workload sha256 bytes)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = kernel_source_sha()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split("#")[0].split()
            if len(parts) == 3 and parts[0] == workload and parts[1] == sha:
                return float(parts[2])
    return None


def copy_probe(nbytes):
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)  # reads 4n bytes, writes 4n bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "launches": 5}))


def affinity_cores():
    """CPU cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count()


def cpu_baseline(probs, target_s):
    """Time the oracle on a bounded sample of the workload, about target_s
    seconds of CPU work: the whole workload, repeated, when one pass is
    shorter than that; otherwise the leading rows of each problem's A with all
    of N and K.  ``cores`` is the number of threads the oracle ran on (its
    OpenMP team: OMP_NUM_THREADS, else every core of the affinity mask)."""
    import oracle

    total_flops = inputs.flops([(p.M, p.N, p.K) for p in probs])
    threads = oracle.num_threads()

    def run(frac):
        flops_done, rows = 0, []
        for p in probs:
            m = min(p.M, max(1, int(round(p.M * frac)))) if p.M > 0 else 0
            rows.append(m)
            if m and p.N:
                oracle.gemm(np.ascontiguousarray(p.A[:m]), np.ascontiguousarray(p.SFA[:m]),
                            p.B, p.SFB, m, p.N, p.K)
                flops_done += 2 * m * p.N * p.K
        return flops_done, rows

    # calibrate on a slice with at least one row per thread
    frac = min(1.0, max(threads / max(1, probs[0].M), 2e9 / total_flops))
    t0 = time.perf_counter()
    f_cal, _ = run(frac)
    rate = f_cal / max(1e-9, time.perf_counter() - t0)
    frac = min(1.0, target_s * rate / total_flops)
    # whole passes (or one partial pass) until about target_s has elapsed
    done, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        f, rows = run(frac)
        done += f
        reps += 1
        dt = time.perf_counter() - t0
        if frac < 1.0 or dt >= target_s:
            break
    if frac >= 1.0:
        sample = "the whole workload, %d pass(es), %.1f s" % (reps, dt)
    else:
        sample = ("leading %s rows of M (all N and K) of each problem: %.3g of the "
                  "workload's flops, %.1f s" % (rows, done / total_flops, dt))
    return {"value": done / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
            "affinity_cores": affinity_cores(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rocm_version():
    """The ROCm release of the image (/opt/rocm/.info/version), or None."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    try:
        with open(os.path.join(rocm, ".info", "version")) as f:
            return f.read().strip()
    except OSError:
        return None


def read_sclk_mhz():
    """The current graphics clock (MHz) from the driver's DPM table in sysfs
    (the entry marked '*' of pp_dpm_sclk), or None."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        if m:
                            return float(m.group(1))
        except OSError:
            continue
    return None


def sample_gfx_clock(run_step, seconds):
    """Graphics clock (MHz, the driver's sysfs DPM table) sampled every 10 ms
    from a helper thread while the calling thread issues run_step() back to
    back for `seconds`.  Returns a summary dict, or one with an "error" when no
    clock can be read."""
    if read_sclk_mhz() is None:
        return {"error": "no readable pp_dpm_sclk"}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            stop.wait(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        run_step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"error": "no clock samples"}
    # the first samples can predate the load: report the busy part
    busy = samples[len(samples) // 5:] or samples
    return {"source": "pp_dpm_sclk", "window_s": seconds, "samples": len(samples),
            "median_mhz": float(np.median(busy)), "min_mhz": float(np.min(busy)),
            "max_mhz": float(np.max(busy))}


class Bench:
    """One workload's operands on the device (several copies), marshalled
    calls, and its timing."""

    def __init__(self, lib, g, b, wl, probs, seed, args):
        import torch
        self.lib, self.g, self.b = lib, g, b
        self.wl, self.probs, self.seed = wl, probs, seed
        self.shapes = [(p.M, p.N, p.K) for p in probs]
        self.flops = inputs.flops(self.shapes)
        self.alg_bytes = inputs.algorithmic_bytes(self.shapes)
        self.blocked = args.scale_layout == "blocked"
        self.pow2 = args.scales == "pow2"
        self.device_table = args.table == "device" and wl.grouped
        dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        sh = self.stream.cuda_stream

        copies = args.copies or max(2, int(np.ceil(2 * CACHE_BYTES / self.alg_bytes)) + 1)
        self.copies = min(copies, 64)
        sets = []
        host = [[torch.from_numpy(x) for x in (p.A, p.SFA, p.B, p.SFB)] for p in probs]
        for _ in range(self.copies):
            one = []
            for p, h in zip(probs, host):
                A, SFA, B, SFB = (x.to(dev) for x in h)
                C = torch.empty((p.M, p.N), dtype=torch.float16, device=dev)
                one.append((A, SFA, B, SFB, C))
            sets.append(one)
        if self.blocked:
            # the scales of every copy moved into the blocked layout, on the
            # device by the library itself
            conv = []
            for one in sets:
                c1 = []
                for (A, SFA, B, SFB, C), p in zip(one, probs):
                    bsa = torch.empty(max(1, g.nvfp4_blocked_scale_bytes(p.M, p.K)), dtype=torch.uint8, device=dev)
                    bsb = torch.empty(max(1, g.nvfp4_blocked_scale_bytes(p.N, p.K)), dtype=torch.uint8, device=dev)
                    g.nvfp4_scales_to_blocked(SFA, bsa, p.M, p.K)
                    g.nvfp4_scales_to_blocked(SFB, bsb, p.N, p.K)
                    c1.append((A, bsa, B, bsb, C))
                conv.append(c1)
            torch.cuda.synchronize()
            sets = conv
        self.sets = sets

        # marshal each set once; a step is then a single C call
        calls = []
        for one in sets:
            if self.device_table:
                rows = [(A, SFA, B, SFB, C, p.M, p.N, p.K) for (A, SFA, B, SFB, C), p in zip(one, probs)]
                table = torch.frombuffer(bytearray(b.problem_table_bytes(rows)), dtype=torch.uint8).to(dev)
                ws = torch.empty(g.nvfp4_group_gemm_device_workspace_bytes(len(one)), dtype=torch.uint8, device=dev)
                tiles = sum(-(-p.M // 128) * -(-p.N // 128) for p in probs if p.M > 0 and p.N > 0)
                calls.append(("device", (table.data_ptr(), len(one), tiles, ws.data_ptr(), ws.numel(), sh),
                              (table, ws)))
            elif not wl.grouped:
                (A, SFA, B, SFB, C), p = one[0], probs[0]
                calls.append(("gemm", (A.data_ptr(), SFA.data_ptr(), B.data_ptr(), SFB.data_ptr(),
                                       C.data_ptr(), p.M, p.N, p.K, sh)))
            else:
                arr = (b.Nvfp4Problem * len(one))()
                for i, ((A, SFA, B, SFB, C), p) in enumerate(zip(one, probs)):
                    arr[i] = b.Nvfp4Problem(A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                                            SFB.data_ptr(), C.data_ptr(), p.M, p.N, p.K)
                calls.append(("group", (arr, len(one), sh)))
        self.calls = calls
        self.gemm_fn = (lib.nvfp4_gemm_blocked if self.blocked else
                        lib.nvfp4_gemm_pow2scale if self.pow2 else lib.nvfp4_gemm)
        self.group_fn = (lib.nvfp4_group_gemm_blocked if self.blocked else
                         lib.nvfp4_group_gemm_pow2scale if self.pow2 else lib.nvfp4_group_gemm)

    def step(self, i):
        kind, a = self.calls[i % len(self.calls)][:2]
        rc = (self.gemm_fn(*a) if kind == "gemm" else self.group_fn(*a) if kind == "group"
              else self.lib.nvfp4_group_gemm_device(*a))
        if rc != 0:
            raise RuntimeError(self.g.status_string(rc))

    def plan(self):
        """The library's plan of the call (host only)."""
        if self.wl.grouped:
            info, _ = self.g.group_gemm_plan(self.shapes)
        else:
            info = self.g.gemm_plan(*self.shapes[0])
        return info

    def run(self, steps, warmup, warmup_seconds=0.0):
        """Time `steps` calls after `warmup` untimed ones (and more untimed
        ones, doubling, until `warmup_seconds` of wall time have passed).
        Returns the timing figures: wall clock of the timed region, the mean
        launch (HIP events on the launch stream around the timed region,
        divided by the steps), a per-launch event-pair distribution, the host
        time of one call, the cache-warm mean launch (same operands every
        step) and the untimed steps run."""
        import torch
        stream = self.stream
        done = settle_warmup(self.step, warmup, warmup_seconds, torch.cuda.synchronize)

        e_start = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e_start.record(stream)
        for i in range(steps):
            self.step(i)
        e_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_s = e_start.elapsed_time(e_end) / 1e3 / steps

        nd = min(steps, 100)
        d0 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        d1 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        host = []
        torch.cuda.synchronize()
        for i in range(nd):
            d0[i].record(stream)
            h0 = time.perf_counter()
            self.step(i)
            host.append(time.perf_counter() - h0)
            d1[i].record(stream)
        torch.cuda.synchronize()
        each_us = np.array([a.elapsed_time(z) for a, z in zip(d0, d1)]) * 1e3

        torch.cuda.synchronize()
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        nwarm = min(steps, 50)
        w0.record(stream)
        for _ in range(nwarm):
            self.step(0)
        w1.record(stream)
        torch.cuda.synchronize()
        warm_s = w0.elapsed_time(w1) / 1e3 / nwarm
        return {"wall_s": wall, "kern_s": kern_s, "each_us": each_us,
                "host_us": float(np.median(host)) * 1e6, "warm_s": warm_s, "warmup_steps_run": done}

    def roofline(self, kern_s):
        """Roofline object of the workload's kernel from its mean launch."""
        kern_tflops = self.flops / kern_s / 1e12
        kern_gbps = self.alg_bytes / kern_s / 1e9
        single = not self.wl.grouped
        traffic = None if (self.blocked or self.device_table or self.pow2) else measured_traffic(self.wl.name)
        if single and self.probs[0].M <= 128 and self.flops / self.alg_bytes < 315:
            # below the fp16 MFMA ridge (2.5 PFLOP/s / 8 TB/s): HBM-bound
            roof = {"bound": "hbm", "achieved": kern_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": kern_gbps / PEAK_HBM_GBPS, "traffic": traffic}
        elif self.pow2:
            # the FP4-MFMA path: its own dtype's peak (fp4 x fp4 MFMA)
            roof = {"bound": "mfma", "achieved": kern_tflops, "peak": PEAK_FP4_TFLOPS,
                    "unit": "TFLOP/s", "frac": kern_tflops / PEAK_FP4_TFLOPS, "traffic": traffic}
        else:
            roof = {"bound": "mfma", "achieved": kern_tflops, "peak": PEAK_FP16_TFLOPS,
                    "unit": "TFLOP/s", "frac": kern_tflops / PEAK_FP16_TFLOPS, "traffic": traffic}
        return roof

    def summary(self, t):
        """Per-workload figures (used for the headline and for each extra)."""
        kern_s = t["kern_s"]
        kern_tflops = self.flops / kern_s / 1e12
        roof = self.roofline(kern_s)
        if self.alg_bytes < 2 ** 20:
            roof["note"] = "latency-bound: too little work to reach either roofline"
        roof["per_launch"] = {
            "flops": self.flops, "algorithmic_bytes": self.alg_bytes,
            "mean_launch_us": kern_s * 1e6,
            "event_pair_us_p10_p50_p90": [float(np.percentile(t["each_us"], q)) for q in (10, 50, 90)],
            "host_call_us_median": t["host_us"]}
        return {
            "workload": self.wl.name, "shapes_MNK": self.shapes, "seed": self.seed,
            "operand_copies": self.copies, "plan": self.plan(),
            "mean_launch_us": kern_s * 1e6, "kernel_tflops": kern_tflops,
            "pct_fp16_peak": 100.0 * kern_tflops / PEAK_FP16_TFLOPS,
            "pct_fp4_peak": 100.0 * kern_tflops / PEAK_FP4_TFLOPS,
            "hbm_gbps": self.alg_bytes / kern_s / 1e9,
            "roofline": roof,
            "warm_cache_us": t["warm_s"] * 1e6,
            "warm_cache_tflops": self.flops / t["warm_s"] / 1e12,
            "warmup_steps_run": t.get("warmup_steps_run"),
        }

    def release(self):
        self.sets = None
        self.calls = None


def settle_warmup(step, warmup, seconds, sync, clock=None):
    """Untimed steps before a timed region: `warmup` of them, then more,
    doubling the count each round (each round ends with `sync`), until
    `seconds` of wall time have passed since the first.  Returns the steps
    run."""
    clock = clock or time.perf_counter
    t0 = clock()
    for i in range(warmup):
        step(i)
    done = warmup
    sync()
    while clock() - t0 < seconds:
        n = max(1, done)
        for j in range(n):
            step(done + j)
        done += n
        sync()
    return done


def workload_spec(index, shape, codes):
    """(Workload, problems, seed) of a named workload or a --shape product."""
    if shape:
        M, N, K = shape
        wl = inputs.Workload("gemm_%dx%dx%d" % (M, N, K), False, "single GEMM M=%d N=%d K=%d" % (M, N, K))
        return wl, inputs.draw_problems(SHAPE_SEED, [(M, N, K)], codes), SHAPE_SEED
    wl = inputs.WORKLOADS[index]
    return wl, inputs.draw_workload(index, codes), inputs.workload_shapes(index)[0]


def compose(args, wl, seed, copies, flops, t, head, extras, cpu, system):
    """The one JSON object bench.py prints."""
    K = args.steps
    return {
        "metric": METRIC,
        "value": flops * K / t["wall_s"] / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": t.get("warmup_steps_run", args.warmup),
        "warmup_min_seconds": args.warmup_seconds,
        "ms_per_step": t["wall_s"] / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1" if args.scales == "pow2" else "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "shapes_MNK": head["shapes_MNK"], "seed": seed,
                   "operand_copies": copies, "scale_layout": args.scale_layout,
                   "scales": args.scales, "table": args.table, "plan": head["plan"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "pct_fp4_peak": head["pct_fp4_peak"],
        "pct_fp16_peak": head["pct_fp16_peak"],
        "hbm_gbps": head["hbm_gbps"],
        "kernel_tflops": head["kernel_tflops"],
        "warm_cache_us": head["warm_cache_us"],
        "warm_cache_tflops": head["warm_cache_tflops"],
        "workloads": extras,
        "system": system,
    }


def main(argv=None):
    args = parse(argv)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    pow2 = args.scales == "pow2"
    if pow2 and args.scale_layout != "plain":
        print("--scales pow2 takes plain-layout scales only", file=sys.stderr)
        sys.exit(2)
    shape = parse_shape(args.shape) if args.shape else None
    if not shape and not 0 <= args.workload < len(inputs.WORKLOADS):
        print("--workload must be in 0..%d" % (len(inputs.WORKLOADS) - 1), file=sys.stderr)
        sys.exit(2)
    head_grouped = False if shape else inputs.WORKLOADS[args.workload].grouped
    if args.table == "device" and (not head_grouped or args.scale_layout != "plain" or pow2):
        print("--table device applies to grouped workloads with general plain-layout scales", file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_gemm_nvfp4_amd as g
    from grouped_gemm_nvfp4_amd import _binding as b

    lib = g.load()
    codes = inputs.POW2_SCALE_CODES if pow2 else inputs.SCALE_CODES

    # the other named workloads first, each released before the next
    extras = {}
    if not shape and not args.no_extras:
        for i, wl in enumerate(inputs.WORKLOADS):
            if i == args.workload:
                continue
            wl_i, probs_i, seed_i = workload_spec(i, None, codes)
            bi = Bench(lib, g, b, wl_i, probs_i, seed_i, args)
            extras[wl_i.name] = bi.summary(bi.run(args.steps, args.warmup, args.warmup_seconds))
            bi.release()
            del bi
            torch.cuda.empty_cache()
            print("timed %s" % wl_i.name, file=sys.stderr, flush=True)

    wl, probs, seed = workload_spec(args.workload, shape, codes)
    bh = Bench(lib, g, b, wl, probs, seed, args)
    t = bh.run(args.steps, args.warmup, args.warmup_seconds)
    head = bh.summary(t)
    clock = sample_gfx_clock(bh.step, args.clock_seconds) if args.clock_seconds > 0 else None

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(probs, args.cpu_seconds)

    system = {"gpu": torch.cuda.get_device_name(0), "rocm": rocm_version(),
              "torch_hip": getattr(torch.version, "hip", None),
              "gfx_clock_under_headline_load": clock,
              "affinity_cores": affinity_cores(),
              "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    out = compose(args, wl, seed, bh.copies, bh.flops, t, head, extras, cpu, system)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
