"""GPU parity for operand transposes, the column bias and the GELU epilogue.

Every configuration runs every operand form (plain and transposed A and B) on
ragged and aligned shapes, with and without bias and GELU, against the oracle's
bound. Small-integer data with transposes (no GELU) must match exactly. The tensor
form must read transposed views in place.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevMatrix, GUARD, say
from workloads import draw, gpt2_linear_set

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def stored(op, x):
    return np.ascontiguousarray(x.T if op else x)


def run_general(config, opA, opB, M, N, K, alpha, a, b, beta, c, bias, act, *, ld_pad=(0, 0, 0),
                offsets=(0, 0, 0)):
    """Run sgemm_general on guarded device buffers; returns (status, C window, checks)."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    As, Bs = stored(opA, a), stored(opB, b)
    lda, ldb, ldc = As.shape[1] + ld_pad[0], Bs.shape[1] + ld_pad[1], N + ld_pad[2]
    dA = DevMatrix(As, As.shape[0], As.shape[1], lda, offsets[0])
    dB = DevMatrix(Bs, Bs.shape[0], Bs.shape[1], ldb, offsets[1])
    dC = DevMatrix(c, M, N, ldc, offsets[2], fill=np.nan if c is None else None)
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    st = sg.sgemm_general(config, opA, opB, M, N, K, alpha, dA.ptr, lda, dB.ptr, ldb, beta, dC.ptr, ldc,
                          dbias, act, torch.cuda.current_stream())
    torch.cuda.synchronize()
    cflat = dC.fetch()
    checks = {"A": dA.unchanged(), "B": dB.unchanged(), "C_outside": dC.outside_unchanged(cflat)}
    return st, dC.window(cflat), checks


def configs():
    """Every data-parallel configuration (the stream-K ones need a workspace and have
    their own tests)."""
    import tiled_fp32_gemm_02_amd as sg
    return [i for i, n in enumerate(sg.configs()) if not n.startswith(("sk_", "sk16_"))]


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 270, 133), (129, 65, 250), (33, 517, 8)])
def test_every_config_every_op(opA, opB, M, N, K):
    rng = np.random.default_rng(M + 3 * N + 7 * K + 11 * opA + 13 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    bias = draw(rng, (N,), "normal")
    for act in (oracle.ACT_NONE, oracle.ACT_GELU_TANH):
        ref, bound = oracle.gemm(opA, opB, M, N, K, 0.75, stored(opA, a), stored(opA, a).shape[1],
                                 stored(opB, b), stored(opB, b).shape[1], -0.5, c, N, bias, act)
        ref0, bound0 = oracle.gemm(opA, opB, M, N, K, 0.75, stored(opA, a), stored(opA, a).shape[1],
                                   stored(opB, b), stored(opB, b).shape[1], -0.5, c, N)
        for cid in configs():
            say(f"op {opA}{opB} act {act} config {cid} {M}x{N}x{K}")
            st, out, checks = run_general(cid, opA, opB, M, N, K, 0.75, a, b, -0.5, c, bias, act)
            assert st == 0 and all(checks.values()), checks
            ok, worst, idx = oracle.within_bound(out, ref, bound)
            assert ok, (cid, act, worst, idx, out[idx], ref[idx])
            # without bias and activation, through the same entry point
            st, out, checks = run_general(cid, opA, opB, M, N, K, 0.75, a, b, -0.5, c, None, oracle.ACT_NONE)
            assert st == 0 and all(checks.values())
            ok, worst, idx = oracle.within_bound(out, ref0, bound0)
            assert ok, (cid, "plain", worst, idx)


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K", [(512, 512, 16), (256, 512, 32), (512, 768, 384), (768, 512, 1024)])
def test_every_config_whole_tiles(opA, opB, M, N, K):
    """Shapes every configuration covers with whole, aligned tiles: the fast kernels
    (including the direct HBM -> LDS copy pipeline) over 1, 2, many and odd counts of
    K-tiles, every operand form, several workgroups."""
    rng = np.random.default_rng(M + 5 * N + 9 * K + 17 * opA + 19 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    ref, bound = oracle.gemm(opA, opB, M, N, K, 1.25, stored(opA, a), stored(opA, a).shape[1],
                             stored(opB, b), stored(opB, b).shape[1], 0.5, c, N)
    for cid in configs():
        say(f"whole tiles op {opA}{opB} config {cid} {M}x{N}x{K}")
        st, out, checks = run_general(cid, opA, opB, M, N, K, 1.25, a, b, 0.5, c, None, oracle.ACT_NONE)
        assert st == 0 and all(checks.values()), checks
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx, out[idx], ref[idx])


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K", [(300, 260, 132), (516, 772, 36), (4, 8, 4), (260, 1028, 1000)])
def test_every_config_aligned_edges(opA, opB, M, N, K):
    """16-byte aligned operands whose tiles cross the M, N and K edges: the aligned edge
    kernels, including direct copies that zero-fill what lies outside the matrix."""
    rng = np.random.default_rng(M + 7 * N + 3 * K + 23 * opA + 29 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    ref, bound = oracle.gemm(opA, opB, M, N, K, -0.75, stored(opA, a), stored(opA, a).shape[1],
                             stored(opB, b), stored(opB, b).shape[1], 1.5, c, N)
    for cid in configs():
        say(f"aligned edges op {opA}{opB} config {cid} {M}x{N}x{K}")
        st, out, checks = run_general(cid, opA, opB, M, N, K, -0.75, a, b, 1.5, c, None, oracle.ACT_NONE)
        assert st == 0 and all(checks.values()), checks
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx, out[idx], ref[idx])


@pytest.mark.parametrize("opA,opB", OPS[1:])
def test_transposes_small_integers_bitwise(opA, opB):
    rng = np.random.default_rng(21 + opA + 2 * opB)
    M, N, K = 131, 97, 203
    a, b, c = (draw(rng, s, "smallint") for s in [(M, K), (K, N), (M, N)])
    bias = draw(rng, (N,), "smallint")
    ref, _ = oracle.gemm(opA, opB, M, N, K, 2.0, stored(opA, a), stored(opA, a).shape[1], stored(opB, b),
                         stored(opB, b).shape[1], -1.0, c, N, bias)
    for cid in configs():
        st, out, checks = run_general(cid, opA, opB, M, N, K, 2.0, a, b, -1.0, c, bias, oracle.ACT_NONE)
        assert st == 0 and all(checks.values())
        assert np.array_equal(out.astype(np.float64), ref), (cid, opA, opB)


@pytest.mark.parametrize("opA,opB", OPS)
def test_ops_unaligned_and_padded(opA, opB):
    rng = np.random.default_rng(31 + opA + 2 * opB)
    M, N, K = 201, 150, 99
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    bias = draw(rng, (N,), "normal")
    ref, bound = oracle.gemm(opA, opB, M, N, K, 1.0, stored(opA, a), stored(opA, a).shape[1], stored(opB, b),
                             stored(opB, b).shape[1], 1.0, c, N, bias, oracle.ACT_GELU_TANH)
    for offsets, ld_pad in [((1, 2, 3), (0, 0, 0)), ((0, 0, 0), (4, 8, 12)), ((0, 0, 0), (1, 3, 5))]:
        for cid in configs():
            st, out, checks = run_general(cid, opA, opB, M, N, K, 1.0, a, b, 1.0, c, bias,
                                          oracle.ACT_GELU_TANH, ld_pad=ld_pad, offsets=offsets)
            assert st == 0 and all(checks.values())
            assert oracle.within_bound(out, ref, bound)[0], (cid, offsets, ld_pad)


@pytest.mark.parametrize("alpha,K", [(0.0, 40), (1.5, 0)])
def test_quick_return_bias_act(alpha, K):
    rng = np.random.default_rng(41)
    M, N = 70, 130
    c = draw(rng, (M, N), "normal")
    bias = draw(rng, (N,), "normal")
    a = np.zeros((M, max(K, 1)), np.float32)
    b = np.zeros((max(K, 1), N), np.float32)
    ref, bound = oracle.gemm(0, 0, M, N, K, alpha, a, max(K, 1), b, N, 0.5, c, N, bias, oracle.ACT_GELU_TANH)
    st, out, checks = run_general(-1, 0, 0, M, N, K, alpha, a[:, :max(K, 1)], b, 0.5, c, bias,
                                  oracle.ACT_GELU_TANH)
    assert st == 0 and checks["C_outside"]
    assert oracle.within_bound(out, ref, bound)[0]


def test_gpt2_mlp_up_with_bias_and_gelu():
    """The GPT-2 MLP's first linear layer with its bias and GELU fused into the product."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    name, X, W = gpt2_linear_set()[1]
    M, K = X.shape
    N = W.shape[1]
    bias = np.float32(0.02) * draw(np.random.default_rng(44), (N,), "normal")
    say(f"{name} + bias + gelu {M}x{N}x{K}")
    dX, dW, db = (torch.from_numpy(v).cuda() for v in (X, W, bias))
    out = sg.gemm(dX, dW, bias=db, act="gelu_tanh")
    torch.cuda.synchronize()
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, X, K, W, N, 0.0, None, N, bias, oracle.ACT_GELU_TANH)
    ok, worst, idx = oracle.within_bound(out.cpu().numpy(), ref, bound)
    assert ok, (worst, idx)
    say(f"worst |err|/bound {worst:.4f}")


def test_tensor_form_reads_transposed_views():
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(51)
    M, N, K = 96, 80, 112
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    At = torch.from_numpy(np.ascontiguousarray(a.T)).cuda()       # stored K x M
    Bt = torch.from_numpy(np.ascontiguousarray(b.T)).cuda()       # stored N x K
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N)
    for A_, B_ in [(At.t(), Bt.t()), (torch.from_numpy(a).cuda(), Bt.t()), (At.t(), torch.from_numpy(b).cuda())]:
        out = sg.gemm(A_, B_)
        torch.cuda.synchronize()
        assert oracle.within_bound(out.cpu().numpy(), ref, bound)[0]
    # a column slice of a transposed view: lda stays the stored row stride
    big = torch.from_numpy(np.ascontiguousarray(np.pad(a.T, ((0, 0), (0, 9))))).cuda()   # K x (M+9)
    out = sg.gemm(big.t()[:M], Bt.t())
    torch.cuda.synchronize()
    assert oracle.within_bound(out.cpu().numpy(), ref, bound)[0]
