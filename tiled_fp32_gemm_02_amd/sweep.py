"""Time kernel configurations on given shapes: the sweep behind the configuration table.

    python -m tiled_fp32_gemm_02_amd.sweep [--shapes M,N,K;...] [--configs all|id,id,...]
                                           [--iters N] [--settle SECONDS] [--beta B] [--workspace]

For every shape and configuration it runs the plain product C = A B + beta C through
sgemm_general_ws on seeded U[-1, 1) inputs (torch's generator, seed 0), lets the clock
settle with untimed calls, then times `iters` back-to-back calls with HIP events on the
launch stream. It prints one line per pair: shape, configuration id and name, mean
microseconds per call and TFLOP/s (2MNK per call). A configuration that the library
rejects for the shape (a stream-K one without --workspace, or one too large) prints its
status instead.

Under `rocprofv3 --kernel-trace --stats` or `--pmc` every configuration's kernel shows
up under its own template name, which is how the counter summaries per configuration
are made. Correctness is the tests' business; this only times.
"""

from __future__ import annotations

import argparse
import time


def parse_shapes(text: str):
    shapes = []
    for part in text.split(";"):
        M, N, K = (int(x) for x in part.split(","))
        shapes.append((M, N, K))
    return shapes


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", default="4096,4096,4096", help="M,N,K;M,N,K;...")
    ap.add_argument("--configs", default="all", help="'all' or comma-separated configuration ids")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.3, help="seconds of untimed calls per pair")
    ap.add_argument("--beta", type=float, default=0.0)
    ap.add_argument("--workspace", action="store_true", help="pass a stream-K workspace")
    args = ap.parse_args(argv)

    import torch
    from . import build as sgbuild
    sgbuild.ensure_built()
    from . import (configs, load, sgemm_general_ws, sgemm_status_string, workspace_for, SGEMM_ACT_NONE,
                   SGEMM_OP_N)
    load()
    if not torch.cuda.is_available():
        raise SystemExit("sweep: needs a GPU")
    dev = torch.device("cuda:0")
    names = configs()
    ids = list(range(len(names))) if args.configs == "all" else [int(x) for x in args.configs.split(",")]
    ws = workspace_for(dev) if args.workspace else None
    ws_ptr, ws_bytes = (ws, ws.numel()) if ws is not None else (None, 0)
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device="cpu").manual_seed(0)
    for M, N, K in parse_shapes(args.shapes):
        A = (torch.rand((M, K), generator=gen) * 2 - 1).to(dev)
        B = (torch.rand((K, N), generator=gen) * 2 - 1).to(dev)
        C = (torch.rand((M, N), generator=gen) * 2 - 1).to(dev)
        flop = 2.0 * M * N * K
        for cid in ids:
            def call():
                return sgemm_general_ws(cid, SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1.0, A, K, B, N, args.beta, C, N,
                                        None, SGEMM_ACT_NONE, ws_ptr, ws_bytes, stream)
            st = call()
            if st != 0:
                print(f"{M}x{N}x{K} {cid:3d} {names[cid]:30s} status {st} ({sgemm_status_string(st)})", flush=True)
                continue
            torch.cuda.synchronize()
            t_end = time.perf_counter() + args.settle
            while time.perf_counter() < t_end:
                for _ in range(4):
                    call()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.iters):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.iters
            print(f"{M}x{N}x{K} {cid:3d} {names[cid]:30s} {us:10.1f} us {flop / us * 1e-6:8.1f} TFLOP/s", flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
