"""GPU parity of every benchmark workload in the launch the benchmark times.

The benchmark hands each product to sgemm_general_ws with a stream-K workspace, lets
the library's cost model choose the configuration (it may pick stream-K; for these
shapes it picks tile kernels) and launches on a stream of its own. These
tests make exactly that call on the workloads' own seeded inputs (and the fused
bias + GELU form of the MLP-up layer) and compare every output entry against the
oracle's bound, not a sample. Each call also checks that A, B and C outside its window
are untouched and that the workspace's tile counters are zero again afterwards.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevMatrix, say
from workloads import WORKLOADS, draw, make

pytestmark = pytest.mark.gpu

COUNTER_WORDS = 16384


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
    return torch.zeros(max(sg.sgemm_workspace_size(-1), 16), dtype=torch.uint8, device="cuda")


def run_as_timed(w, A, B, C, bias, act, ws):
    """One call as the benchmark makes it; returns (config name, C window, checks)."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    dA = DevMatrix(A, w.M, w.K, w.lda_, 0)
    dB = DevMatrix(B, w.K, w.N, w.ldb_, 0)
    dC = DevMatrix(C, w.M, w.N, w.ldc_, 0, fill=np.nan if C is None else None)
    cfg = sg.sgemm_select_config_ws(w.M, w.N, w.K, w.alpha, dA.ptr, w.lda_, dB.ptr, w.ldb_, dC.ptr, w.ldc_,
                                    ws.numel())
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    stream = torch.cuda.Stream()
    st = sg.sgemm_general_ws(-1, sg.SGEMM_OP_N, sg.SGEMM_OP_N, w.M, w.N, w.K, w.alpha, dA.ptr, w.lda_, dB.ptr,
                             w.ldb_, w.beta, dC.ptr, w.ldc_, dbias, act, ws, ws.numel(), int(stream.cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, sg.sgemm_status_string(st)
    flat = dC.fetch()
    checks = {"A": dA.unchanged(), "B": dB.unchanged(), "C_outside": dC.outside_unchanged(flat)}
    counters = ws[:4 * COUNTER_WORDS].view(dtype=torch.int32)
    checks["counters_clear"] = int(counters.abs().sum().item()) == 0
    return sg.sgemm_config_name(cfg), dC.window(flat), checks


@pytest.mark.parametrize("name", ["sq256", "sq1024", "ragged", "sq4096", "gpt2_qkv", "gpt2_mlp_up",
                                  "gpt2_mlp_down", "gpt2_mlp_up_gelu"])
def test_workload_as_timed(name, ws):
    import tiled_fp32_gemm_02_amd as sg
    fused = name == "gpt2_mlp_up_gelu"
    w = WORKLOADS["gpt2_mlp_up" if fused else name]
    A, B, C = make(w)
    # the fused layer's bias is drawn as the benchmark draws it
    bias = draw(np.random.default_rng(w.seed + 1000), (w.N,), "normal002") if fused else None
    act = sg.SGEMM_ACT_GELU_TANH if fused else sg.SGEMM_ACT_NONE
    say(f"workload {name} as timed: {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta}")
    cfg_name, out, checks = run_as_timed(w, A, B, C, bias, act, ws)
    say(f"workload {name}: configuration {cfg_name}")
    assert all(checks.values()), (name, cfg_name, checks)
    ref, bound = oracle.gemm(0, 0, w.M, w.N, w.K, w.alpha, A, w.lda_, B, w.ldb_, w.beta, C, w.ldc_, bias,
                             oracle.ACT_GELU_TANH if fused else oracle.ACT_NONE)
    ok, worst, idx = oracle.within_bound(out, ref, bound)
    assert ok, f"{name} ({cfg_name}): max |err|/bound = {worst} at {idx}: got {out[idx]}, oracle {ref[idx]}"
    say(f"workload {name}: max |err|/bound = {worst:.4f}")


def test_timed_configurations(ws):
    """What the cost model picks for the timed launches, with a workspace: the measured
    winners of the sweep. 16x16-block tiles for GPT-2 QKV (64 x 64 with stream-K: two whole
    rounds of 256 tiles, the last 64 tiles shared by every CU), MLP-up (64 x 64, wave tiles of
    16 x 64), 1024^3 (64 x 64 x 64) and 256^3 (16 x 16, all of K in one K-tile); the 32 x 32
    tile of 32x32 blocks for MLP-down; the 256 x 256 tile at 4096^3 (one tile per CU)."""
    import tiled_fp32_gemm_02_amd as sg
    picks = {}
    for name in ["gpt2_qkv", "gpt2_mlp_up", "gpt2_mlp_down", "sq256", "sq1024", "sq4096"]:
        w = WORKLOADS[name]
        picks[name] = sg.sgemm_config_name(sg.sgemm_select_config_ws(
            w.M, w.N, w.K, w.alpha, ws.data_ptr(), w.lda_, ws.data_ptr(), w.ldb_, ws.data_ptr(), w.ldc_,
            ws.numel()))
    say(f"timed configurations: {picks}")
    assert picks["gpt2_qkv"] == "sk16_64x64x32_w4x1k1d"
    assert picks["gpt2_mlp_up"] == "mfma16_64x64x32_w4x1k1d"
    assert picks["gpt2_mlp_down"] == "mfma_32x32x64_w1x1k4d" and picks["sq256"] == "mfma16_16x16x256_w1x1k4d"
    assert picks["sq1024"] == "mfma16_64x64x64_w4x1k2d"
    assert picks["sq4096"] == "mfma_256x256x32_w2x4d"
