#!/usr/bin/env python3
"""Benchmark of the fp32 GEMM hot path on one MI355X.

A step is one call of ``sgemm`` (host dispatch + one kernel) on the workload,
with every input already resident in HBM. The default workload is the 4096^3
product with alpha = 1.5, beta = 0.5 (A, B, C uniform on [-1, 1), seed 2); the
timed calls run in place on C, which stays bounded (C <- 1.5 AB + 0.5 C tends
to 3 AB).

Prints one JSON line: the metric (TFLOP/s, 2*M*N*K flops per call), the
roofline of the kernel (flops per launch / mean launch time from HIP events on
the launch stream, against the MI355X fp32 matrix peak of 157.3 TFLOP/s), and
the CPU oracle timed on a bounded sample of the same product on this host.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--config ID]
                    [--no-cpu-baseline] [--copy-probe]

``--copy-probe`` instead runs a plain device-to-device copy of a known size, the
calibration run for the HBM byte counters.
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
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3          # MI355X dense fp32 (matrix and vector), AMD's published figure
CSRC = os.path.join(ROOT, "tiled_fp32_gemm_02_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 of the kernel sources with comments and whitespace removed, so the
    recorded counters stay valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".hpp", ".inc")):
            continue
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_traffic(workload: str, config_name: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source and the same workload and configuration; else None."""
    path = os.path.join(ROOT, "profiles", f"{config_name}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if (vals.get("kernel_source_sha256") != kernel_source_hash() or vals.get("workload") != workload
                or vals.get("config") != config_name):
            return None
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, A, B, C, target_s: float):
    """Time the CPU oracle on the first R rows of the product (R chosen from a pilot
    run so the sample takes about `target_s` seconds). Returns the JSON object."""
    import oracle
    N, K = w.N, w.K

    def run(rows):
        t0 = time.perf_counter()
        oracle.sgemm(rows, N, K, w.alpha, A, w.lda_, B, w.ldb_, w.beta, C, w.ldc_, with_bound=False)
        return time.perf_counter() - t0

    pilot_rows = min(w.M, 16)
    t_pilot = run(pilot_rows)
    rows = int(min(w.M, max(pilot_rows, round(target_s * pilot_rows / max(t_pilot, 1e-6)))))
    t = run(rows)
    flops = 2.0 * rows * N * K
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": (f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} product ({rows}x{N}x{K}, "
                   f"{flops / 1e9:.1f} GFLOP, fp64 accumulation, {t:.1f} s wall)"),
    }


def copy_probe(steps: int):
    """Plain device copy of 256 MiB, `steps` times: the reference for the byte counters."""
    import torch
    n = 64 * 1024 * 1024
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "launches": steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sq4096")
    ap.add_argument("--config", type=int, default=-1, help="force a kernel configuration id")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the product would shard by rows of A and C; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.steps)
        return

    import torch
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    from workloads import WORKLOADS, make, flops

    w = WORKLOADS[args.workload]
    A, B, C = make(w)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C).to(dev) if C is not None else torch.empty((w.M, w.ldc_), device=dev)
    C0 = dC.clone()
    cfg = args.config if args.config >= 0 else sg.sgemm_select_config(
        w.M, w.N, w.K, w.alpha, dA, w.lda_, dB, w.ldb_, dC, w.ldc_)
    cfg_name = sg.sgemm_config_name(cfg)
    stream = torch.cuda.Stream(device=dev)
    s_handle = int(stream.cuda_stream)

    def step():
        st = sg.sgemm_ex(args.config, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                         w.beta, dC.data_ptr(), w.ldc_, s_handle)
        if st != 0:
            raise RuntimeError(f"sgemm failed: {sg.sgemm_status_string(st)}")

    # One checked call on a fresh C: sampled entries against the oracle.
    log(f"bench: workload {w.name} {w.M}x{w.N}x{w.K} config {cfg} {cfg_name}")
    step()
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    rng = np.random.default_rng(12345)
    rows = np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 254)])
    cols = np.concatenate([[0, w.N - 1], rng.integers(0, w.N, 254)])
    import oracle
    ref, bound = oracle.sgemm_entries(w.M, w.N, w.K, w.alpha, A, w.lda_, B, w.ldb_, w.beta, C, w.ldc_,
                                      rows, cols)
    ok, worst, _ = oracle.within_bound(out[rows, cols], ref, bound)
    if not ok:
        raise SystemExit(f"bench: result outside the oracle bound (max |err|/bound = {worst})")
    log(f"bench: checked {rows.size} sampled entries, max |err|/bound = {worst:.3f}")
    dC.copy_(C0)
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_s = t1 - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    fl = flops(w.M, w.N, w.K)
    value = fl * args.steps / wall_s / 1e12
    achieved = fl / (kernel_ms * 1e-3) / 1e12
    log(f"bench: {args.steps} steps in {wall_s * 1e3:.2f} ms wall; mean kernel {kernel_ms * 1e3:.1f} us")

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": ("FP32 SGEMM TFLOP/s at M=N=K=4096 and fraction of MI355X FP32 peak" if w.name == "sq4096"
                   else f"FP32 SGEMM TFLOP/s ({w.name}) and fraction of MI355X FP32 peak"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
                   "inputs": w.note, "kernel": cfg_name, "parallelism": "none (one GPU)"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": recorded_traffic(w.name, cfg_name),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "check": {"sampled_entries": int(rows.size), "max_err_over_bound": round(worst, 4)},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w, A, B, C, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
