"""GPU parity for general-stride operands (sgemm_strided and the tensor form over it).

The GPT-2 post's kernel takes operands with dynamic strides, so sliced and transposed
views run without copies ("GPU Target - GPT-2 on the GPU", section "Tiled matrix
multiplication"). Each case lays the operands out as strided views inside larger device
buffers of random values, runs the product in place, and checks:
  - the M x N window against the oracle, computed on dense copies of the same views,
    elementwise within the bound (bitwise for small-integer data, where every sum is
    exact in fp32);
  - every buffer float outside the C window unchanged, bitwise.
Layouts cover every route: the general-stride kernel (no unit stride, repeated rows or
columns, overlapping rows, a column-major C with a bias), the transposed product (a
column-major C without bias) and the stored-matrix kernels (views that are row-major or
transposed after all), plus the quick returns on a strided C.
"""

import numpy as np
import pytest

import oracle
from gpu_util import say
from workloads import draw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def _span(shape, strides, offset):
    return offset + sum((n - 1) * s for n, s in zip(shape, strides) if n > 0) + 1


def _run(M, N, K, a_layout, b_layout, c_layout, *, alpha=1.5, beta=0.5, bias=False, act=0, dist="normal",
         seed=0, raw=True):
    """Run one product on strided views. A layout is (strides, offset). Each operand's
    whole buffer is drawn from `dist` (C's from U[-1, 1)) and the views read it in place,
    so repeated and overlapping entries hold one value; the oracle sees dense copies of
    the views. Returns (C window, dense A, dense B, oracle ref, bound)."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(seed)
    views = []
    for (strides, off), shape, kind in ((a_layout, (M, K), dist), (b_layout, (K, N), dist),
                                        (c_layout, (M, N), "uniform")):
        buf = torch.from_numpy(draw(rng, (_span(shape, strides, off) + 16,), kind)).cuda()
        views.append((buf, torch.as_strided(buf, shape, strides, off)))
    (bufA, A), (bufB, B), (bufC, C) = views
    bvec = draw(rng, (N,), "normal") if bias else None
    a_dense, b_dense, c_dense = A.cpu().numpy(), B.cpu().numpy(), C.cpu().numpy()
    before = bufC.cpu().numpy().copy()
    dbias = torch.from_numpy(bvec).cuda() if bias else None
    say(f"strided {M}x{N}x{K} A{a_layout} B{b_layout} C{c_layout} alpha {alpha} beta {beta} bias {bias} "
        f"act {act} raw {raw}")
    if raw:
        st = sg.sgemm_strided(M, N, K, alpha, A, A.stride(0), A.stride(1), B, B.stride(0), B.stride(1), beta, C,
                              C.stride(0), C.stride(1), dbias, act, torch.cuda.current_stream())
        assert st == 0, (st, sg.sgemm_status_string(st))
    else:
        sg.gemm(A, B, C, alpha=alpha, beta=beta, bias=dbias, act=("gelu_tanh" if act else None))
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    after = bufC.cpu().numpy()
    # every float of C's buffer outside the window is unchanged
    mask = np.ones(after.shape, bool)
    off = c_layout[1]
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    mask[off + rows * c_layout[0][0] + cols * c_layout[0][1]] = False
    assert np.array_equal(after[mask].view(np.uint32), before[mask].view(np.uint32)), "C buffer changed outside"
    ref, bound = oracle.gemm(0, 0, M, N, K, alpha, a_dense, K, b_dense, N, beta, c_dense, N, bvec, act)
    return out, a_dense, b_dense, ref, bound


def _check(out, ref, bound):
    ok, worst, idx = oracle.within_bound(out, ref, bound)
    assert ok, (worst, idx, out[idx], ref[idx])


# (A layout, B layout, C layout) as ((row stride, column stride), offset), for M, N, K below
GENERAL = [
    # every other column of A, every third row and second column of B, a C with strides (2N+1, 2)
    lambda M, N, K: (((2 * K + 3, 2), 1), ((3 * N * 2, 2), 0), (((2 * N + 1), 2), 3)),
    # A stored column-major with a padded column stride and a column step: neither stride 1
    lambda M, N, K: (((3, 3 * M + 5), 2), ((N + 4, 1), 1), ((N, 1), 0)),
    # a repeated row of A (row stride 0) and a repeated column of B (column stride 0)
    lambda M, N, K: (((0, 1), 0), ((1, 0), 0), ((N + 1, 1), 0)),
    # rows of A that overlap in memory (row stride 3 < K), and a column-major C with a bias
    lambda M, N, K: (((3, 1), 0), ((N, 1), 0), ((1, M + 2), 5)),
]


@pytest.mark.parametrize("M,N,K", [(70, 45, 33), (300, 260, 200), (1, 37, 19), (53, 1, 41), (64, 64, 1)])
@pytest.mark.parametrize("case", range(len(GENERAL)))
def test_general_strides(M, N, K, case):
    la, lb, lc = GENERAL[case](M, N, K)
    bias = case == 3
    out, _, _, ref, bound = _run(M, N, K, la, lb, lc, bias=bias, seed=case * 7 + M)
    _check(out, ref, bound)


@pytest.mark.parametrize("M,N,K", [(96, 80, 64), (131, 67, 257)])
def test_small_integers_exact(M, N, K):
    """Every partial sum exact in fp32: the general-stride kernel equals the brute force bitwise."""
    for case in (0, 1):
        la, lb, lc = GENERAL[case](M, N, K)
        out, a, b, _, _ = _run(M, N, K, la, lb, lc, alpha=1.0, beta=0.0, dist="smallint", seed=M + case)
        exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float32)
        assert np.array_equal(out, exact)


def test_column_major_c_runs_as_the_transposed_product():
    """No bias: C^T = B^T A^T on the stored-matrix kernels; with GELU too."""
    M, N, K = 200, 150, 96
    for act in (0, 1):
        out, _, _, ref, bound = _run(M, N, K, ((K, 1), 0), ((N, 1), 0), ((1, M), 0), act=act, seed=40 + act)
        _check(out, ref, bound)


def test_stored_layouts_through_the_general_entry():
    """Row-major and transposed views passed with explicit strides take the stored-matrix
    kernels; the result is the same product."""
    M, N, K = 257, 190, 129
    for la, lb in ((((K + 3, 1), 0), ((N, 1), 2)), (((1, M + 1), 0), ((1, K), 1))):
        out, _, _, ref, bound = _run(M, N, K, la, lb, ((N + 5, 1), 1), bias=True, act=1, seed=50)
        _check(out, ref, bound)


@pytest.mark.parametrize("alpha,K", [(0.0, 33), (1.5, 0)])
def test_quick_returns_on_a_strided_c(alpha, K):
    """alpha == 0 or K == 0: C <- act(beta*C + bias) through C's strides, A and B unread."""
    M, N = 45, 38
    lc = ((2 * N + 1, 2), 3)
    out, _, _, ref, bound = _run(M, N, K, ((max(K, 1) * 2, 2), 0), ((2 * N, 2), 0), lc, alpha=alpha,
                                 beta=0.5, bias=True, act=1, seed=60)
    _check(out, ref, bound)


def test_tensor_form_on_general_views():
    """gemm() takes views with no unit stride (slices with steps, expanded dimensions) in place."""
    M, N, K = 120, 90, 70
    for case in range(len(GENERAL)):
        la, lb, lc = GENERAL[case](M, N, K)
        out, _, _, ref, bound = _run(M, N, K, la, lb, lc, bias=case == 3, act=case % 2, seed=70 + case,
                                     raw=False)
        _check(out, ref, bound)
