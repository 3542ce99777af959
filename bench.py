#!/usr/bin/env python3
"""Throughput of the NVFP4 GEMM / grouped GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]

One step is one call of the library (nvfp4_gemm for a single product,
nvfp4_group_gemm for a grouped one) over one set of synthetic operands that
already sit in device memory.  The default workload is the small-M,
bandwidth-bound product M=64 N=7168 K=16384; ``--workload`` picks another of
the named workloads in grouped_gemm_nvfp4_amd/inputs.py.

Steps cycle over several identical copies of the operands whose total size
exceeds the 256 MiB Infinity Cache plus the L2s, so each step reads its
operands from HBM rather than from a cache warmed by the previous step.

Prints one JSON line: TFLOPS = sum 2*M*N*K / time, the roofline of the kernel
(algorithmic bytes or flops per launch over its mean launch duration: the
timed region measured with HIP events on the launch stream, divided by the
number of steps), and the CPU oracle's throughput on a bounded sample of the
same workload.  The roofline's "traffic" (HBM bytes per launch from the
FETCH_SIZE and WRITE_SIZE counters) comes from profiles/hbm_traffic.txt and is
reported only while the kernel sources it was measured on are unchanged.

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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1,
                    help="index into grouped_gemm_nvfp4_amd.inputs.WORKLOADS")
    ap.add_argument("--shape", default=None, metavar="M,N,K",
                    help="time one GEMM of these sizes (seeded inputs, seed %d) instead of a "
                         "named workload" % SHAPE_SEED)
    ap.add_argument("--copies", type=int, default=0,
                    help="operand copies to cycle over (0: enough to exceed the caches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0: skip)")
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
    return ap.parse_args()


KERNEL_DIR = os.path.join(ROOT, "grouped_gemm_nvfp4_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


SHAPE_SEED = 2000  # inputs of a --shape run


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


def cpu_baseline(probs, target_s):
    """Time the oracle on a bounded sample of the workload, about target_s
    seconds of CPU work: the whole workload, repeated, when one pass is
    shorter than that; otherwise the leading rows of each problem's A with all
    of N and K."""
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


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_gemm_nvfp4_amd as g
    from grouped_gemm_nvfp4_amd import _binding as b

    lib = g.load()
    pow2 = args.scales == "pow2"
    if pow2 and args.scale_layout != "plain":
        print("--scales pow2 takes plain-layout scales only", file=sys.stderr)
        sys.exit(2)
    codes = inputs.POW2_SCALE_CODES if pow2 else inputs.SCALE_CODES
    if args.shape:
        M, N, K = parse_shape(args.shape)
        wl = inputs.Workload("gemm_%dx%dx%d" % (M, N, K), False, "single GEMM M=%d N=%d K=%d" % (M, N, K))
        seed = SHAPE_SEED
        probs = inputs.draw_problems(seed, [(M, N, K)], codes)
    else:
        wl = inputs.WORKLOADS[args.workload]
        seed = inputs.workload_shapes(args.workload)[0]
        probs = inputs.draw_workload(args.workload, codes)
    shapes = [(p.M, p.N, p.K) for p in probs]
    flops = inputs.flops(shapes)
    alg_bytes = inputs.algorithmic_bytes(shapes)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    copies = args.copies or max(2, int(np.ceil(2 * CACHE_BYTES / alg_bytes)) + 1)
    copies = min(copies, 64)
    sets = []
    host = [[torch.from_numpy(x) for x in (p.A, p.SFA, p.B, p.SFB)] for p in probs]
    for _ in range(copies):
        one = []
        for p, h in zip(probs, host):
            A, SFA, B, SFB = (x.to(dev) for x in h)
            C = torch.empty((p.M, p.N), dtype=torch.float16, device=dev)
            one.append((A, SFA, B, SFB, C))
        sets.append(one)

    blocked = args.scale_layout == "blocked"
    if blocked:
        # the scales of every copy moved into the blocked layout, on the device
        # by the library itself
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

    device_table = args.table == "device" and wl.grouped
    if args.table == "device" and (not wl.grouped or blocked or pow2):
        print("--table device applies to grouped workloads with general plain-layout scales", file=sys.stderr)
        sys.exit(2)
    # marshal each set once; a step is then a single C call
    calls = []
    for one in sets:
        if device_table:
            rows = [(A, SFA, B, SFB, C, p.M, p.N, p.K) for (A, SFA, B, SFB, C), p in zip(one, probs)]
            table = torch.frombuffer(bytearray(b.problem_table_bytes(rows)), dtype=torch.uint8).to(dev)
            ws = torch.empty(g.nvfp4_group_gemm_device_workspace_bytes(len(one)), dtype=torch.uint8, device=dev)
            tiles = sum(-(-p.M // 128) * -(-p.N // 128) for p in probs if p.M > 0 and p.N > 0)
            calls.append(("device", (table.data_ptr(), len(one), tiles, ws.data_ptr(), ws.numel(), sh),
                          (table, ws)))
            continue
        if not wl.grouped:
            (A, SFA, B, SFB, C), p = one[0], probs[0]
            args_c = (A.data_ptr(), SFA.data_ptr(), B.data_ptr(), SFB.data_ptr(),
                      C.data_ptr(), p.M, p.N, p.K, sh)
            calls.append(("gemm", args_c))
        else:
            arr = (b.Nvfp4Problem * len(one))()
            for i, ((A, SFA, B, SFB, C), p) in enumerate(zip(one, probs)):
                arr[i] = b.Nvfp4Problem(A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                                        SFB.data_ptr(), C.data_ptr(), p.M, p.N, p.K)
            calls.append(("group", (arr, len(one), sh)))
    gemm_fn = lib.nvfp4_gemm_blocked if blocked else lib.nvfp4_gemm_pow2scale if pow2 else lib.nvfp4_gemm
    group_fn = (lib.nvfp4_group_gemm_blocked if blocked else
                lib.nvfp4_group_gemm_pow2scale if pow2 else lib.nvfp4_group_gemm)

    def step(i):
        kind, a = calls[i % len(calls)][:2]
        rc = (gemm_fn(*a) if kind == "gemm" else group_fn(*a) if kind == "group"
              else lib.nvfp4_group_gemm_device(*a))
        if rc != 0:
            raise RuntimeError(g.status_string(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(K):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_s = e_start.elapsed_time(e_end) / 1e3 / K

    # per-launch distribution (a separate pass: an event pair around each
    # call), and the host time of one call (enqueue only, no synchronisation)
    nd = min(K, 100)
    d0 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
    d1 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
    host = []
    torch.cuda.synchronize()
    for i in range(nd):
        d0[i].record(stream)
        h0 = time.perf_counter()
        step(i)
        host.append(time.perf_counter() - h0)
        d1[i].record(stream)
    torch.cuda.synchronize()
    each_us = np.array([a.elapsed_time(z) for a, z in zip(d0, d1)]) * 1e3
    host_us = float(np.median(host)) * 1e6

    # same operands every step (cache-warm), for context only
    torch.cuda.synchronize()
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    nwarm = min(K, 50)
    w0.record(stream)
    for _ in range(nwarm):
        step(0)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_s = w0.elapsed_time(w1) / 1e3 / nwarm

    value = flops * K / wall / 1e12
    kern_tflops = flops / kern_s / 1e12
    kern_gbps = alg_bytes / kern_s / 1e9
    small_m = (not wl.grouped) and probs[0].M <= 128
    if small_m:
        roof = {"bound": "hbm", "achieved": kern_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": kern_gbps / PEAK_HBM_GBPS,
                "traffic": None if blocked else measured_traffic(wl.name)}
    elif pow2:
        # the FP4-MFMA path: its own dtype's peak (fp4 x fp4 MFMA)
        roof = {"bound": "mfma", "achieved": kern_tflops, "peak": PEAK_FP4_TFLOPS,
                "unit": "TFLOP/s", "frac": kern_tflops / PEAK_FP4_TFLOPS, "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": kern_tflops, "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": kern_tflops / PEAK_FP16_TFLOPS,
                "traffic": None if blocked or device_table else measured_traffic(wl.name)}
    roof["per_launch"] = {"flops": flops, "algorithmic_bytes": alg_bytes,
                          "mean_launch_us": kern_s * 1e6,
                          "event_pair_us_p10_p50_p90": [float(np.percentile(each_us, q)) for q in (10, 50, 90)],
                          "host_call_us_median": host_us}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(probs, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1" if pow2 else "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "shapes_MNK": shapes, "seed": seed,
                   "operand_copies": copies, "scale_layout": args.scale_layout,
                   "scales": args.scales, "table": args.table},
        "roofline": roof,
        "cpu_baseline": cpu,
        "pct_fp4_peak": 100.0 * kern_tflops / PEAK_FP4_TFLOPS,
        "pct_fp16_peak": 100.0 * kern_tflops / PEAK_FP16_TFLOPS,
        "hbm_gbps": kern_gbps,
        "kernel_tflops": kern_tflops,
        "warm_cache_us": warm_s * 1e6,
        "warm_cache_tflops": flops / warm_s / 1e12,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
