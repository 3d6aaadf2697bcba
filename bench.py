#!/usr/bin/env python3
"""Benchmark of the fp32 GEMM hot path on one MI355X.

A step is one call of the library (host dispatch + one kernel) on the workload,
with every input already resident in HBM. The call passes a stream-K workspace,
allocated and zeroed before timing, so the library may pick a stream-K kernel.
The default workload is the 4096^3 product with alpha = 1.5, beta = 0.5 (A, B, C
uniform on [-1, 1), seed 2); the timed calls run in place on C, which stays
bounded (C <- 1.5 AB + 0.5 C tends to 3 AB).

Prints one JSON line: the metric (TFLOP/s, 2*M*N*K flops per call), the
roofline of the kernel (flops per launch / mean launch time from HIP events on
the launch stream, against the MI355X fp32 matrix peak of 157.3 TFLOP/s), and
the CPU oracle timed on a bounded sample of the same product on this host.

    python bench.py [--steps K] [--warmup W] [--settle-seconds S] [--workload NAME]
                    [--config ID|NAME] [--no-cpu-baseline] [--copy-probe]

Before the W warm-up steps the step runs back to back, untimed, for S seconds
(default 1): the GPU's clock ramps up over the first tens of milliseconds of
load, and a short warm-up alone times the kernel partly at the lower clock. The
timed region is exactly K steps, bracketed by synchronisations; an event is
recorded on the launch stream between steps, so the line also carries the
median, minimum and 90th percentile of the per-step times. The shader clock is
read from sysfs before and after the timed steps where the driver exposes it.

``--workload gpt2_seq`` times the three GPT-2-small linears (QKV, MLP up, MLP
down) in that order as one step: total flops over total time.
``--workload gpt2_attn`` times attention's two per-head batched products (12 heads
of Q K^T / 8 with K transposed in place, then P V with the heads side by side), as
one step.
``--workload gpt2_mlp_up_gelu`` is the MLP-up layer with its bias and tanh GELU
fused into the product's final write (bias ~ 0.02 N(0,1), drawn from seed 4 + 1000);
flops are counted as 2MNK, as for the plain product.

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


def read_sclk():
    """Current shader clock in MHz from the amdgpu driver's sysfs table (the entry
    marked '*'), or None where it is not readable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().replace("mhz", "").strip(" *"))
        except (OSError, ValueError, IndexError):
            continue
    return None


# The sources that define the matrix-core kernels and which variant a launch runs: the
# kernel templates, the launchers, their instantiation and the configuration table. Host
# dispatch (sgemm_api.hip) and the vector-ALU kernels do not change a matrix-core kernel.
MFMA_KERNEL_SOURCES = ("sgemm_kernels.hpp", "sgemm_launch.hpp", "sgemm_launch_impl.hpp", "sgemm_inst.hip",
                       "sgemm_configs.inc")


def kernel_source_hash() -> str:
    """sha256 of the matrix-core kernel sources with comments and whitespace removed, so
    the recorded counters stay valid across comment-only edits and host-side changes."""
    import re
    h = hashlib.sha256()
    for name in MFMA_KERNEL_SOURCES:
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def host_cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or ''."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def tile_dims(config_name: str):
    """(BM, BN) of a configuration from its name (e.g. mfma_256x256x32_w2x4d -> (256, 256);
    tile16 -> (16, 16))."""
    import re
    if config_name == "tile16":
        return 16, 16
    m = re.search(r"_(\d+)x(\d+)x\d+", config_name)
    if not m:
        raise ValueError(f"no tile shape in configuration name {config_name!r}")
    return int(m.group(1)), int(m.group(2))


def lds_fill_bytes(M: int, N: int, K: int, config_name: str) -> float:
    """Bytes the tiles copy from memory into LDS (or registers) per launch: each BM x BN tile
    reads a BM-row panel of A and a BN-column panel of B over all of K, so
    4 M N K (1/BM + 1/BN) in total. The L2 caches serve what HBM does not (the measured
    FETCH_SIZE is the part that misses)."""
    bm, bn = tile_dims(config_name)
    return 4.0 * M * N * K * (1.0 / bm + 1.0 / bn)


def register_tile(config_name: str):
    """(TM, TN): the register tile whose rows and columns each LDS read feeds, from the
    configuration's name. For the matrix-core kernels it is the wave's tile
    (BM/WGM x BN/WGN); for the vector-ALU kernel the thread's 8 x 8 micro-tile; for the
    16x16 kernel one output per thread."""
    import re
    if config_name == "tile16":
        return 1, 1
    m = re.search(r"_t(\d+)x(\d+)$", config_name)
    if m:
        return int(m.group(1)), int(m.group(2))
    m = re.search(r"_(\d+)x(\d+)x\d+_w(\d+)x(\d+)", config_name)
    if not m:
        raise ValueError(f"no wave grid in configuration name {config_name!r}")
    bm, bn, wm, wn = (int(x) for x in m.groups())
    return bm // wm, bn // wn


def lds_read_bytes(M: int, N: int, K: int, config_name: str) -> float:
    """Bytes read from LDS into registers per launch: for every k, each TM x TN register
    tile reads its TM values of op(A) and TN values of op(B), so 4 M N K (1/TM + 1/TN) in
    total (AutoMine++ #4's count for its register tile, "Let's use registers")."""
    tm, tn = register_tile(config_name)
    return 4.0 * M * N * K * (1.0 / tm + 1.0 / tn)


def peak_at_clock(cus, sclk_mhz):
    """The fp32 matrix peak at a measured shader clock: CUs x 256 flop/clk x sclk, in TFLOP/s
    (None when the clock was not readable)."""
    if not cus or not sclk_mhz:
        return None
    return cus * 256 * sclk_mhz * 1e6 / 1e12


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


class LinearProblem:
    """One plain product of the workload table (optionally with bias + tanh GELU), with
    its host inputs, device copies and the configuration the library picks."""

    def __init__(self, sg, torch, dev, w, config, ws, fused):
        from workloads import draw, make
        self.sg, self.w, self.name, self.note = sg, w, w.name, w.note
        self.M, self.N, self.K, self.batch = w.M, w.N, w.K, 1
        self.A, self.B, self.C = make(w)
        self.dA = torch.from_numpy(self.A).to(dev)
        self.dB = torch.from_numpy(self.B).to(dev)
        self.dC = (torch.from_numpy(self.C).to(dev) if self.C is not None
                   else torch.empty((w.M, w.ldc_), device=dev))
        self.C0 = self.dC.clone()
        self.config, self.ws = config, ws
        self.cfg = config if config >= 0 else sg.sgemm_select_config_ws(
            w.M, w.N, w.K, w.alpha, self.dA, w.lda_, self.dB, w.ldb_, self.dC, w.ldc_, ws.numel())
        self.cfg_name = sg.sgemm_config_name(self.cfg)
        self.bias = draw(np.random.default_rng(w.seed + 1000), (w.N,), "normal002") if fused else None
        self.dbias = torch.from_numpy(self.bias).to(dev) if fused else None
        self.act = sg.SGEMM_ACT_GELU_TANH if fused else sg.SGEMM_ACT_NONE

    def launch(self, stream_handle):
        w, sg = self.w, self.sg
        st = sg.sgemm_general_ws(self.config, sg.SGEMM_OP_N, sg.SGEMM_OP_N, w.M, w.N, w.K, w.alpha,
                                 self.dA.data_ptr(), w.lda_, self.dB.data_ptr(), w.ldb_, w.beta,
                                 self.dC.data_ptr(), w.ldc_, self.dbias, self.act, self.ws.data_ptr(),
                                 self.ws.numel(), stream_handle)
        if st != 0:
            raise RuntimeError(f"sgemm failed: {sg.sgemm_status_string(st)}")

    def check(self, oracle):
        """256 sampled entries (the corners included) against the oracle: (worst, count)."""
        w = self.w
        out = self.dC.cpu().numpy()
        rng = np.random.default_rng(12345)
        rows = np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 254)])
        cols = np.concatenate([[0, w.N - 1], rng.integers(0, w.N, 254)])
        ref, bound = oracle.gemm_entries(0, 0, w.M, w.N, w.K, w.alpha, self.A, w.lda_, self.B, w.ldb_, w.beta,
                                         self.C, w.ldc_, rows, cols, bias=self.bias, act=self.act)
        ok, worst, _ = oracle.within_bound(out[rows, cols], ref, bound)
        if not ok:
            raise SystemExit(f"bench: {w.name} outside the oracle bound (max |err|/bound = {worst})")
        self.dC.copy_(self.C0)
        return worst, rows.size

    def cpu(self, oracle, rows):
        """Seconds for the oracle on the first `rows` rows of the product."""
        w = self.w
        t0 = time.perf_counter()
        oracle.gemm(0, 0, rows, w.N, w.K, w.alpha, self.A, w.lda_, self.B, w.ldb_, w.beta, self.C, w.ldc_,
                    self.bias, self.act, with_bound=False)
        return time.perf_counter() - t0

    def describe(self):
        return {"name": self.name, "M": self.M, "N": self.N, "K": self.K, "kernel": self.cfg_name}


class BatchedProblem:
    """One strided-batched product (workloads.BatchedGemm) over shared device buffers, with
    the operand forms read in place."""

    def __init__(self, sg, torch, dev, prob, bufs, dbufs, config):
        self.sg, self.p, self.name, self.note = sg, prob, prob.name, prob.note
        self.M, self.N, self.K, self.batch = prob.M, prob.N, prob.K, prob.batch
        self.bufs, self.dbufs = bufs, dbufs
        self.dC = torch.zeros(prob.c_rows * prob.c_cols, device=dev)
        self.config = config
        self.cfg = config if config >= 0 else sg.sgemm_select_config_general(
            prob.opA, prob.opB, prob.M, prob.N, prob.K, prob.alpha, self._ptr(prob.a, prob.a_off), prob.lda,
            prob.sA, self._ptr(prob.b, prob.b_off), prob.ldb, prob.sB, self.dC.data_ptr() + 4 * prob.c_off,
            prob.ldc, prob.sC, prob.batch)
        self.cfg_name = sg.sgemm_config_name(self.cfg)

    def _ptr(self, name, off):
        return self.dbufs[name].data_ptr() + 4 * off

    def launch(self, stream_handle):
        p, sg = self.p, self.sg
        st = sg.sgemm_strided_batched_general(self.config, p.opA, p.opB, p.M, p.N, p.K, p.alpha,
                                              self._ptr(p.a, p.a_off), p.lda, p.sA, self._ptr(p.b, p.b_off),
                                              p.ldb, p.sB, 0.0, self.dC.data_ptr() + 4 * p.c_off, p.ldc, p.sC,
                                              None, sg.SGEMM_ACT_NONE, p.batch, stream_handle)
        if st != 0:
            raise RuntimeError(f"sgemm_strided_batched_general failed: {sg.sgemm_status_string(st)}")

    def _operands(self, b):
        p = self.p
        a = self.bufs[p.a].reshape(-1)[p.a_off + b * p.sA:]
        bb = self.bufs[p.b].reshape(-1)[p.b_off + b * p.sB:]
        return a, bb

    def check(self, oracle):
        """256 sampled entries, spread over the batches (the first and last batch's corners
        included), against the oracle: (worst, count)."""
        p = self.p
        out = self.dC.cpu().numpy()
        rng = np.random.default_rng(12345)
        bs = np.concatenate([[0, p.batch - 1], rng.integers(0, p.batch, 254)])
        rows = np.concatenate([[0, p.M - 1], rng.integers(0, p.M, 254)])
        cols = np.concatenate([[0, p.N - 1], rng.integers(0, p.N, 254)])
        worst = 0.0
        for b in np.unique(bs):
            sel = bs == b
            a, bb = self._operands(int(b))
            ref, bound = oracle.gemm_entries(p.opA, p.opB, p.M, p.N, p.K, p.alpha, a, p.lda, bb, p.ldb, 0.0, None,
                                             p.ldc, rows[sel], cols[sel])
            got = out[p.c_off + int(b) * p.sC + rows[sel] * p.ldc + cols[sel]]
            ok, wb, _ = oracle.within_bound(got, ref, bound)
            if not ok:
                raise SystemExit(f"bench: {p.name} batch {b} outside the oracle bound (max |err|/bound = {wb})")
            worst = max(worst, wb)
        return worst, bs.size

    def cpu(self, oracle, rows):
        """Seconds for the oracle on the first `rows` rows of every batch."""
        p = self.p
        t0 = time.perf_counter()
        for b in range(p.batch):
            a, bb = self._operands(b)
            oracle.gemm(p.opA, p.opB, rows, p.N, p.K, p.alpha, a, p.lda, bb, p.ldb, 0.0, None, p.ldc,
                        with_bound=False)
        return time.perf_counter() - t0

    def describe(self):
        p = self.p
        return {"name": p.name, "batch": p.batch, "M": p.M, "N": p.N, "K": p.K, "opA": "NT"[p.opA],
                "opB": "NT"[p.opB], "kernel": self.cfg_name}


def cpu_baseline(probs, target_s: float):
    """Time the CPU oracle on the first rows of each product of the step (the same
    fraction of every product's rows, chosen from a pilot run so that the sample
    takes about `target_s` seconds). Returns the JSON object."""
    import oracle

    pilot = [min(p.M, 16) for p in probs]
    t_pilot = sum(p.cpu(oracle, r) for p, r in zip(probs, pilot))
    frac = min(1.0, target_s / max(t_pilot, 1e-6) * sum(pilot) / sum(p.M for p in probs))
    rows = [int(min(p.M, max(r, round(frac * p.M)))) for p, r in zip(probs, pilot)]
    t = sum(p.cpu(oracle, r) for p, r in zip(probs, rows))
    flops = sum(2.0 * r * p.N * p.K * p.batch for p, r in zip(probs, rows))
    what = "; ".join(f"rows 0..{r - 1} of {'each of the %d ' % p.batch if p.batch > 1 else 'the '}"
                     f"{p.M}x{p.N}x{p.K} product{'s' if p.batch > 1 else ''}" for p, r in zip(probs, rows))
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{what} ({flops / 1e9:.1f} GFLOP, fp64 accumulation, {t:.1f} s wall)",
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
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed back-to-back steps before the warm-up, for the clock to ramp")
    ap.add_argument("--workload", default="sq4096")
    ap.add_argument("--config", default="-1", help="force a kernel configuration (id or name)")
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
    import oracle
    from workloads import WORKLOADS, flops

    if args.config.lstrip("-").isdigit():
        args.config = int(args.config)
    elif args.config in sg.configs():
        args.config = sg.configs().index(args.config)
    else:
        raise SystemExit(f"bench: no configuration named {args.config!r}; see tiled_fp32_gemm_02_amd.configs()")
    fused = args.workload == "gpt2_mlp_up_gelu"
    dev = torch.device("cuda:0")
    # The stream-K workspace (zero-filled once, outside the timed region): the library
    # picks stream-K configurations where its cost model favours them.
    ws = torch.zeros(max(sg.sgemm_workspace_size(-1), 16), dtype=torch.uint8, device=dev)
    if args.workload == "gpt2_attn":
        from workloads import attention_products, gpt2_attention_set
        bufs = gpt2_attention_set()
        dbufs = {k: torch.from_numpy(v).to(dev) for k, v in bufs.items()}
        probs = [BatchedProblem(sg, torch, dev, pr, bufs, dbufs, args.config) for pr in attention_products()]
    else:
        names = (["gpt2_qkv", "gpt2_mlp_up", "gpt2_mlp_down"] if args.workload == "gpt2_seq"
                 else ["gpt2_mlp_up"] if fused else [args.workload])
        if any(n not in WORKLOADS for n in names):
            raise SystemExit(f"bench: unknown workload {args.workload!r}")
        probs = [LinearProblem(sg, torch, dev, WORKLOADS[n], args.config, ws, fused) for n in names]
    stream = torch.cuda.Stream(device=dev)
    s_handle = int(stream.cuda_stream)

    def step():
        for p in probs:
            p.launch(s_handle)

    # One checked call on a fresh C: sampled entries against the oracle.
    for p in probs:
        log(f"bench: workload {p.name} {p.batch} x {p.M}x{p.N}x{p.K} config {p.cfg} {p.cfg_name}")
    step()
    torch.cuda.synchronize()
    worst_all, checked = 0.0, 0
    for p in probs:
        worst, n = p.check(oracle)
        worst_all, checked = max(worst_all, worst), checked + n
    log(f"bench: checked {checked} sampled entries, max |err|/bound = {worst_all:.3f}")
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        t_end = time.perf_counter() + args.settle_seconds
        settle = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            settle += 8
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        sclk_before = read_sclk()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sclk_after = read_sclk()
    wall_s = t1 - t0
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])    # ms
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    fl = sum(flops(p.M, p.N, p.K) * p.batch for p in probs)
    value = fl * args.steps / wall_s / 1e12
    achieved = fl / (kernel_ms * 1e-3) / 1e12
    log(f"bench: {settle} settle steps, {args.warmup} warm-up; {args.steps} steps in {wall_s * 1e3:.2f} ms wall; "
        f"mean step {kernel_ms * 1e3:.1f} us (events)")

    props = torch.cuda.get_device_properties(dev)
    clocks = [c for c in (sclk_before, sclk_after) if c]
    sclk_mean = sum(clocks) / len(clocks) if clocks else None
    peak_sclk = peak_at_clock(props.multi_processor_count, sclk_mean)
    if len(probs) == 1:
        p0, w0 = probs[0], probs[0].w
        config = {"workload": args.workload, "M": w0.M, "N": w0.N, "K": w0.K, "alpha": w0.alpha, "beta": w0.beta,
                  "inputs": w0.note, "kernel": p0.cfg_name, "parallelism": "none (one GPU)"}
        if fused:
            config["epilogue"] = "bias + tanh GELU"
        metric = ("FP32 SGEMM TFLOP/s at M=N=K=4096 and fraction of MI355X FP32 peak" if w0.name == "sq4096"
                  else f"FP32 SGEMM TFLOP/s ({args.workload}) and fraction of MI355X FP32 peak")
        traffic = recorded_traffic(args.workload, p0.cfg_name)
    else:
        config = {"workload": args.workload, "sequence": [p.describe() for p in probs],
                  "inputs": "; ".join(p.note for p in probs), "parallelism": "none (one GPU)"}
        metric = f"FP32 SGEMM TFLOP/s ({args.workload}: the products in sequence) and fraction of MI355X FP32 peak"
        traffic = None
    line = {
        "metric": metric,
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
        "config": config,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": traffic,
            "peak_at_sclk": round(peak_sclk, 2) if peak_sclk else None,
            "frac_at_sclk": round(achieved / peak_sclk, 4) if peak_sclk else None,
            "sclk_mhz": round(sclk_mean, 1) if sclk_mean else None,
        },
        "timing": {"settle_steps": settle, "step_us_median": round(float(np.median(per_step)) * 1e3, 2),
                   "step_us_min": round(float(per_step.min()) * 1e3, 2),
                   "step_us_p90": round(float(np.percentile(per_step, 90)) * 1e3, 2),
                   "sclk_mhz_before": sclk_before, "sclk_mhz_after": sclk_after},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "hip": torch.version.hip,
                   "host_cpu": host_cpu_model(), "host_threads": len(os.sched_getaffinity(0))},
        "check": {"sampled_entries": int(checked), "max_err_over_bound": round(worst_all, 4)},
        "tile_traffic": {"global_to_lds_bytes": round(sum(p.batch * lds_fill_bytes(p.M, p.N, p.K, p.cfg_name)
                                                          for p in probs)),
                         "lds_to_register_bytes": round(sum(p.batch * lds_read_bytes(p.M, p.N, p.K, p.cfg_name)
                                                            for p in probs)),
                         "model": "per step: 4*M*N*K*(1/BM + 1/BN) for the tiles' operand panels into LDS; "
                                  "4*M*N*K*(1/TM + 1/TN) from LDS into each TM x TN wave (or thread) tile"},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(probs, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
