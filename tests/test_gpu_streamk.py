"""GPU parity of the stream-K configurations (C-ABI entry point with a workspace).

Every stream-K configuration runs every operand form on shapes that cover the ways
the work can split: fewer K-tile steps than compute units, tiles shared
by two or several workgroups, ranges that hold whole tiles between partial ones, edge
tiles in M, N and K, bias + GELU, more tiles than compute units (whole tiles first, the
last round's tiles shared), and unaligned operands (the direct-copy configurations' own
kernel, register-staged ones the data-parallel kernel of the tile). Results are checked
against the oracle's bound, must be bitwise
identical from run to run, and the workspace's tile counters must be zero again after
every call.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevMatrix, say
from workloads import draw

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
COUNTER_WORDS = 16384        # per-tile counters at the start of the workspace


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


@pytest.fixture(scope="module")
def ws():
    import torch
    import tiled_fp32_gemm_02_amd as sg
    n = sg.sgemm_workspace_size(-1)
    assert n > 4 * COUNTER_WORDS
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def sk_ids():
    import tiled_fp32_gemm_02_amd as sg
    return [i for i, n in enumerate(sg.configs()) if n.startswith(("sk_", "sk16_"))]


def stored(op, x):
    return np.ascontiguousarray(x.T if op else x)


def run_ws(config, opA, opB, M, N, K, alpha, a, b, beta, c, bias, act, ws, offsets=(0, 0, 0)):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    As, Bs = stored(opA, a), stored(opB, b)
    dA = DevMatrix(As, As.shape[0], As.shape[1], As.shape[1], offsets[0])
    dB = DevMatrix(Bs, Bs.shape[0], Bs.shape[1], Bs.shape[1], offsets[1])
    dC = DevMatrix(c, M, N, N, offsets[2])
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    st = sg.sgemm_general_ws(config, opA, opB, M, N, K, alpha, dA.ptr, As.shape[1], dB.ptr, Bs.shape[1], beta,
                             dC.ptr, N, dbias, act, ws, ws.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    flat = dC.fetch()
    checks = {"A": dA.unchanged(), "B": dB.unchanged(), "C_outside": dC.outside_unchanged(flat)}
    return st, dC.window(flat), checks


def counters_clear(ws):
    return int(ws[:4 * COUNTER_WORDS].view(dtype=__import__("torch").int32).abs().sum().item()) == 0


SHAPES = [
    (100, 132, 64),          # fewer K-tile steps than compute units: one workgroup per step
    (100, 130, 70),          # unaligned: direct-copy configurations keep their kernel
    (256, 512, 256),         # each tile shared by several workgroups
    (1024, 768, 1024),       # GPT-2 MLP-down-like: 48..96 tiles, K long
    (1028, 772, 516),        # aligned, with M, N and K edges
    (2048, 1024, 128),       # more tiles than workgroups: whole tiles between partial ones
    (1028, 1540, 516),       # more tiles than compute units: whole tiles, then the last round shared
    (1000, 1537, 777),       # the same, unaligned (4-byte aligned rows), edges in M, N and K
]


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_stream_k_every_config(opA, opB, M, N, K, ws):
    rng = np.random.default_rng(M + 3 * N + 5 * K + 7 * opA + 11 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    ref, bound = oracle.gemm(opA, opB, M, N, K, 1.25, stored(opA, a), stored(opA, a).shape[1], stored(opB, b),
                             stored(opB, b).shape[1], -0.5, c, N)
    for cid in sk_ids():
        say(f"stream-K op {opA}{opB} config {cid} {M}x{N}x{K}")
        st, out, checks = run_ws(cid, opA, opB, M, N, K, 1.25, a, b, -0.5, c, None, oracle.ACT_NONE, ws)
        assert st == 0 and all(checks.values()), (st, checks)
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx, out[idx], ref[idx])
        assert counters_clear(ws)


@pytest.mark.parametrize("M,N,K", [(1024, 2304, 768), (300, 260, 132)])
def test_stream_k_bias_gelu(M, N, K, ws):
    rng = np.random.default_rng(M + N + K)
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal002")
    bias = draw(rng, (N,), "normal")
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias, oracle.ACT_GELU_TANH)
    for cid in sk_ids():
        say(f"stream-K bias+gelu config {cid} {M}x{N}x{K}")
        st, out, checks = run_ws(cid, 0, 0, M, N, K, 1.0, a, b, 0.0, np.zeros((M, N), np.float32), bias,
                                 oracle.ACT_GELU_TANH, ws)
        assert st == 0 and all(checks.values())
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx)


def test_stream_k_bitwise_reproducible(ws):
    M, N, K = 1024, 768, 3072
    rng = np.random.default_rng(5)
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    zero = np.zeros((M, N), np.float32)
    for cid in sk_ids():
        say(f"stream-K reproducibility config {cid}")
        outs = [run_ws(cid, 0, 0, M, N, K, 1.0, a, b, 0.0, zero, None, 0, ws)[1] for _ in range(3)]
        assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_stream_k_small_integers_exact(ws):
    # every partial sum is an integer below 2^24: any order of summation is exact
    M, N, K = 257, 300, 640
    rng = np.random.default_rng(9)
    a = rng.integers(-8, 9, (M, K)).astype(np.float32)
    b = rng.integers(-8, 9, (K, N)).astype(np.float32)
    exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float32)
    for cid in sk_ids():
        for opA, opB in OPS:
            say(f"stream-K exact op {opA}{opB} config {cid}")
            st, out, _ = run_ws(cid, opA, opB, M, N, K, 1.0, a, b, 0.0, np.zeros((M, N), np.float32), None, 0,
                                ws)
            assert st == 0 and np.array_equal(out, exact)


def test_stream_k_unaligned_operands(ws):
    # offsets of 1..3 floats: the data-parallel kernel of the same tile runs
    M, N, K = 513, 515, 517
    rng = np.random.default_rng(13)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    ref, bound = oracle.gemm(0, 0, M, N, K, 0.5, a, K, b, N, 2.0, c, N)
    for cid in sk_ids():
        say(f"stream-K unaligned config {cid}")
        st, out, checks = run_ws(cid, 0, 0, M, N, K, 0.5, a, b, 2.0, c, None, 0, ws, offsets=(1, 2, 3))
        assert st == 0 and all(checks.values())
        assert oracle.within_bound(out, ref, bound)[0]


def test_auto_choice_with_workspace(ws):
    import tiled_fp32_gemm_02_amd as sg
    names = sg.configs()
    picks = {}
    for M, N, K in [(1536, 1536, 1536), (2560, 2560, 2560), (4096, 4096, 4096)]:
        cid = sg.sgemm_select_config_ws(M, N, K, 1.0, ws.data_ptr(), K, ws.data_ptr(), N, ws.data_ptr(), N,
                                        ws.numel())
        picks[(M, N, K)] = names[cid]
    assert picks[(4096, 4096, 4096)] == "mfma_256x256x32_w2x4d"       # one whole tile per CU already
    assert picks[(2560, 2560, 2560)].startswith(("sk_", "sk16_"))   # long K, a sparse last round of tiles
    # 576 tiles of 64 x 64: two whole rounds, the last 64 tiles shared by all CUs (60 us measured,
    # against 66 for 768 tiles of 32 x 96 without stream-K)
    assert picks[(1536, 1536, 1536)] == "sk16_64x64x32_w4x1k1d"


def test_tensor_form_uses_the_workspace():
    """The tensor form passes its cached workspace, so a shape the cost model sends to
    stream-K (512 x 512 x 8192: 16 tiles of 128 x 128, K long) gets it; without the workspace
    the same call runs a tile kernel."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(17)
    M, N, K = 512, 512, 8192
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal002")
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    ws = sg.workspace_for(A.device)
    assert sg.sgemm_config_name(sg.sgemm_select_config_ws(M, N, K, 1.0, A, K, B, N, A, N, ws.numel())).startswith(("sk_", "sk16_"))
    say("stream-K through the tensor form")
    C = sg.gemm(A, B)
    C2 = sg.gemm(A, B, workspace=None)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N)
    assert oracle.within_bound(C.cpu().numpy(), ref, bound)[0]
    assert oracle.within_bound(C2.cpu().numpy(), ref, bound)[0]
    assert counters_clear(ws)


def test_tensor_form_on_a_side_stream_with_a_fresh_workspace(monkeypatch):
    """gemm(..., stream=s) on a stream other than the current one, with the workspace
    cache empty: the buffer's zero fill is queued on the current stream, and must be
    complete before the stream-K kernel on s reads its counters. Checked elementwise
    against the oracle, and the counters are zero again afterwards."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    monkeypatch.setattr(sg, "_workspaces", {})
    rng = np.random.default_rng(23)
    M, N, K = 512, 512, 8192
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal002")
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    torch.cuda.synchronize()
    ws_bytes = sg.sgemm_workspace_size(-1)
    assert sg.sgemm_config_name(sg.sgemm_select_config_ws(M, N, K, 1.0, A, K, B, N, A, N, ws_bytes)).startswith(("sk_", "sk16_"))
    side = torch.cuda.Stream()
    # reuse of a freed allocation: leave nonzero bytes where the workspace may land
    junk = torch.full((sg.sgemm_workspace_size(-1) // 4 + 16,), -1, dtype=torch.int32, device="cuda")
    del junk
    say("stream-K through the tensor form on a side stream, fresh workspace")
    C = sg.gemm(A, B, stream=side)
    side.synchronize()
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N)
    ok, worst, idx = oracle.within_bound(C.cpu().numpy(), ref, bound)
    assert ok, (worst, idx)
    ws = sg._workspaces[(A.device.index, int(side.cuda_stream))]
    assert counters_clear(ws)
