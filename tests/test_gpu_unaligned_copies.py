"""GPU parity of the direct copies on rows that are only 4-byte aligned.

There the direct-copy kernels keep their 16-byte copies, issued from 4-byte aligned
addresses, so a chunk that crosses the end of a row brings floats of the next row (or of
the row-stride gap) into the tile. Along m or n those land in tile rows or columns past the
matrix edge; the K-tile that holds the end of K is copied float by float instead. These cases
fill every row-stride gap and guard band with NaN, so any float from outside the matrix that
reached a result would turn it into NaN. Each direct-copy configuration runs every operand
form on shapes with row strides of exactly 4 and 5 floats, one to three columns, K inside one
K-tile and K ending a few floats into a K-tile, checked elementwise against the oracle; A and
B must be untouched, and C outside its window too. Row strides under 4 floats take the
register-staged kernel, which the same cases cover.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevMatrix, say
from workloads import draw

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
# (M, N, K, padding added to the stored row length of A, B and C)
SHAPES = [
    (37, 5, 9, (0, 0, 0)),        # strides 9 and 5; K inside one K-tile
    (70, 1, 13, (0, 3, 0)),       # one column of B with a row stride of exactly 4
    (65, 3, 4, (1, 1, 0)),        # strides 5 and 4
    (33, 130, 37, (0, 1, 3)),     # K ending five floats into its second K-tile of 32
    (3, 67, 200, (1, 0, 2)),      # three rows, long K ending eight floats into a K-tile
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def direct_copy_configs():
    import tiled_fp32_gemm_02_amd as sg
    return [i for i, n in enumerate(sg.configs()) if n.startswith(("mfma_", "mfma16_")) and n.endswith("d")]


def stored(op, x):
    return np.ascontiguousarray(x.T if op else x)


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K,pad", SHAPES)
def test_direct_copies_on_unaligned_rows(opA, opB, M, N, K, pad):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(M + 5 * N + 11 * K + 3 * opA + 7 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    As, Bs = stored(opA, a), stored(opB, b)
    lda, ldb, ldc = As.shape[1] + pad[0], Bs.shape[1] + pad[1], N + pad[2]
    ref, bound = oracle.gemm(opA, opB, M, N, K, 1.25, As, As.shape[1], Bs, Bs.shape[1], -0.5, c, N)
    for cid in direct_copy_configs():
        say(f"unaligned direct copies config {cid} op {opA}{opB} {M}x{N}x{K} lda {lda} ldb {ldb} ldc {ldc}")
        dA = DevMatrix(As, As.shape[0], As.shape[1], lda, 1, gap=np.nan)
        dB = DevMatrix(Bs, Bs.shape[0], Bs.shape[1], ldb, 2, gap=np.nan)
        dC = DevMatrix(c, M, N, ldc, 3, gap=np.nan)
        st = sg.sgemm_general(cid, opA, opB, M, N, K, 1.25, dA.ptr, lda, dB.ptr, ldb, -0.5, dC.ptr, ldc, None, 0,
                              torch.cuda.current_stream())
        torch.cuda.synchronize()
        flat = dC.fetch()
        assert st == 0, (cid, st)
        assert dA.unchanged() and dB.unchanged() and dC.outside_unchanged(flat), cid
        out = dC.window(flat)
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx, out[idx], ref[idx])
