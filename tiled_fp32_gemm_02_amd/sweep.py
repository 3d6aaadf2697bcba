"""Time kernel configurations on given shapes: the sweep behind the configuration table.

    python -m tiled_fp32_gemm_02_amd.sweep [--shapes M,N,K;...] [--configs all|id,id,...]
                                           [--iters N] [--settle SECONDS] [--beta B] [--workspace]
                                           [--batch B] [--opa n|t] [--opb n|t]

For every shape and configuration it runs the product C = op(A) op(B) + beta C through
sgemm_general_ws (or, with --batch above 1, sgemm_strided_batched_general over packed
matrices) on seeded U[-1, 1) inputs (torch's generator, seed 0), lets the clock settle
with untimed calls, then times `iters` back-to-back calls with HIP events on the launch
stream. It prints one line per pair: shape (prefixed with the batch and operand forms
when not the plain product), configuration id and name, mean microseconds per call and
TFLOP/s (2MNK per product). A configuration that the library
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
    ap.add_argument("--batch", type=int, default=1,
                    help="strided-batched products of packed matrices (no stream-K)")
    ap.add_argument("--opa", choices=("n", "t"), default="n", help="read A as stored or transposed")
    ap.add_argument("--opb", choices=("n", "t"), default="n", help="read B as stored or transposed")
    args = ap.parse_args(argv)

    import torch
    from . import build as sgbuild
    sgbuild.ensure_built()
    from . import (configs, load, sgemm_general_ws, sgemm_status_string, sgemm_strided_batched_general,
                   workspace_for, SGEMM_ACT_NONE)
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
    opa, opb = int(args.opa == "t"), int(args.opb == "t")
    bsz = args.batch
    for M, N, K in parse_shapes(args.shapes):
        ar, ac = (K, M) if opa else (M, K)         # A and B as stored
        br, bc = (N, K) if opb else (K, N)
        A = (torch.rand((bsz, ar, ac), generator=gen) * 2 - 1).to(dev)
        B = (torch.rand((bsz, br, bc), generator=gen) * 2 - 1).to(dev)
        C = (torch.rand((bsz, M, N), generator=gen) * 2 - 1).to(dev)
        flop = 2.0 * M * N * K * bsz
        for cid in ids:
            def call():
                if bsz > 1:
                    return sgemm_strided_batched_general(cid, opa, opb, M, N, K, 1.0, A, ac, ar * ac, B, bc,
                                                         br * bc, args.beta, C, N, M * N, None, SGEMM_ACT_NONE, bsz,
                                                         stream)
                return sgemm_general_ws(cid, opa, opb, M, N, K, 1.0, A, ac, B, bc, args.beta, C, N,
                                        None, SGEMM_ACT_NONE, ws_ptr, ws_bytes, stream)
            st = call()
            if st != 0:
                print(f"{bsz}x{M}x{N}x{K} {cid:3d} {names[cid]:30s} status {st} ({sgemm_status_string(st)})",
                      flush=True)
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
            shape = f"{bsz}x{M}x{N}x{K}{args.opa}{args.opb}" if bsz > 1 or opa or opb else f"{M}x{N}x{K}"
            print(f"{shape} {cid:3d} {names[cid]:30s} {us:10.1f} us {flop / us * 1e-6:8.1f} TFLOP/s", flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
