"""GPU parity of the fringe columns of the data-parallel matrix kernels.

When N mod BN = r is 1..8 and the whole tiles number at least 256 (over the batch), the tile
grid stops at column N - r and extra workgroups compute the last r columns, two rows of C
each, their threads splitting K. These cases run every data-parallel matrix configuration in every
operand form on a shape of 2 x 128 whole tiles plus r fringe columns (fewer than 256 fringe
workgroups, so one round of them even where one workgroup fills a CU's LDS), with the full epilogue
(alpha, beta, and on some of them a bias and the GELU), and check against the oracle every row
of the fringe columns and of the last whole column before them, and a random sample of the
rest. Row-stride gaps and guard bands hold NaN, so a load outside the matrices would show; A
and B must be untouched, and C outside its window too. The launch shape is checked to be the
fringe one, so a change of rule cannot silently route these cases around the fringe path.
Further cases: batched products, long K against the full oracle, and M and K multiples of the
tile on aligned rows, where the tiles beside the fringe run the kernel without edge tests.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DevMatrix, say
from workloads import draw

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
FRINGES = [1, 5, 8, 3, 2, 7]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def matrix_configs():
    import tiled_fp32_gemm_02_amd as sg
    return [i for i, n in enumerate(sg.configs()) if n.startswith(("mfma_", "mfma16_"))]


def stored(op, x):
    return np.ascontiguousarray(x.T if op else x)


def tile_of(cid):
    import tiled_fp32_gemm_02_amd as sg
    d = sg.describe(cid)
    bm, bn, _ = (int(v) for v in d["tile"].split("x"))
    return bm, bn, int(d["threads"])


def check_entries(out, opA, opB, M, N, K, alpha, As, Bs, beta, c, bias, act, rows, cols, what):
    ref, bound = oracle.gemm_entries(opA, opB, M, N, K, alpha, As, As.shape[1], Bs, Bs.shape[1], beta, c, N,
                                     rows, cols, bias=bias, act=act)
    ok, worst, idx = oracle.within_bound(out[rows, cols], ref, bound)
    assert ok, (what, worst, int(rows[idx]), int(cols[idx]), out[rows[idx], cols[idx]], ref[idx])


def fringe_samples(rng, M, N, r):
    """Every row of the last r + 1 columns, and 512 random entries."""
    rr, cc = np.meshgrid(np.arange(M), np.arange(N - r - 1, N), indexing="ij")
    rows = np.concatenate([rr.reshape(-1), rng.integers(0, M, 512)])
    cols = np.concatenate([cc.reshape(-1), rng.integers(0, N, 512)])
    return rows, cols


@pytest.mark.parametrize("opA,opB", OPS)
def test_fringe_columns_every_configuration(opA, opB):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    for n, cid in enumerate(matrix_configs()):
        bm, bn, threads = tile_of(cid)
        r = FRINGES[n % len(FRINGES)]
        # K ragged and within the three memory round trips a fringe workgroup may take
        steps = 4 if r <= 2 else 2 if r <= 4 else 1
        M, N, K = 2 * bm - 3, 128 * bn + r, min((45, 300, 1100)[n % 3], 3 * threads * steps - 5)
        st, grid, _ = sg.sgemm_launch_shape(cid, M, N, K)
        assert st == 0 and grid[0] == 256 + -(-M // 2), (cid, grid)
        rng = np.random.default_rng(cid + 100 * opA + 1000 * opB)
        a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
        bias = draw(rng, (N,), "normal") if n % 2 else None
        act = sg.SGEMM_ACT_GELU_TANH if n % 3 == 1 else sg.SGEMM_ACT_NONE
        As, Bs = stored(opA, a), stored(opB, b)
        lda, ldb, ldc = As.shape[1] + 1, Bs.shape[1] + 2, N + 3
        say(f"fringe config {cid} op {opA}{opB} {M}x{N}x{K} r {r} bias {bias is not None} act {act}")
        dA = DevMatrix(As, As.shape[0], As.shape[1], lda, 1, gap=np.nan)
        dB = DevMatrix(Bs, Bs.shape[0], Bs.shape[1], ldb, 2, gap=np.nan)
        dC = DevMatrix(c, M, N, ldc, 3, gap=np.nan)
        dbias = torch.from_numpy(bias).cuda() if bias is not None else None
        st = sg.sgemm_general(cid, opA, opB, M, N, K, 1.25, dA.ptr, lda, dB.ptr, ldb, -0.5, dC.ptr, ldc, dbias, act,
                              torch.cuda.current_stream())
        torch.cuda.synchronize()
        flat = dC.fetch()
        assert st == 0, (cid, st)
        assert dA.unchanged() and dB.unchanged() and dC.outside_unchanged(flat), cid
        out = dC.window(flat)
        rows, cols = fringe_samples(rng, M, N, r)
        check_entries(out, opA, opB, M, N, K, 1.25, As, Bs, -0.5, c, bias, act, rows, cols, cid)


@pytest.mark.parametrize("name", ["mfma16_64x64x32_w4x1k1d", "mfma16_32x64x64_w2x1k2d", "mfma_64x64x32_w2x2k2"])
@pytest.mark.parametrize("opB", [0, 1])
def test_fringe_columns_batched(name, opB):
    """Two products of 8 x 16 whole tiles each (256 over the batch) and 3 fringe columns:
    the fringe workgroups of each product read and write that product's matrices."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    names = sg.configs()
    if name not in names:
        pytest.skip(f"{name} not built")
    cid = names.index(name)
    bm, bn, _ = tile_of(cid)
    batch, M, N, K = 2, 8 * bm - 1, 16 * bn + 3, 203
    rng = np.random.default_rng(cid + 7 * opB)
    a = draw(rng, (batch, M, K), "normal")
    b = draw(rng, (batch, K, N), "normal")
    c = draw(rng, (batch, M, N), "uniform")
    bs = np.ascontiguousarray(b.transpose(0, 2, 1)) if opB else b
    ldb = bs.shape[2]
    dA = torch.from_numpy(a).cuda()
    dB = torch.from_numpy(bs).cuda()
    dC = torch.from_numpy(c).cuda()
    say(f"fringe batched {name} opB {opB} {batch}x{M}x{N}x{K}")
    st = sg.sgemm_strided_batched_general(cid, 0, opB, M, N, K, 0.75, dA.data_ptr(), K, M * K, dB.data_ptr(), ldb,
                                          K * N, 0.5, dC.data_ptr(), N, M * N, None, 0, batch,
                                          torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == 0, st
    out = dC.cpu().numpy()
    for z in range(batch):
        rows, cols = fringe_samples(rng, M, N, 3)
        check_entries(out[z], 0, opB, M, N, K, 0.75, a[z], bs[z], 0.5, c[z], None, sg.SGEMM_ACT_NONE, rows, cols,
                      (name, z))


def test_fringe_columns_long_k_workload_shape():
    """The 1000 x 1537 x 777 product with 4-byte aligned rows on the 64 x 64 tile (one fringe
    column, 384 whole tiles) and a K of 2100 on the 32 x 64 tile (several steps of the
    fringe's k loop): every entry against the oracle."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    names = sg.configs()
    for name, (M, N, K) in [("mfma16_64x64x32_w4x1k1d", (1000, 1537, 777)),
                            ("mfma16_32x64x64_w2x1k2d", (1000, 1537, 2100))]:
        cid = names.index(name)
        rng = np.random.default_rng(K)
        a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
        say(f"fringe full check {name} {M}x{N}x{K}")
        dA = DevMatrix(a, M, K, K, 1, gap=np.nan)
        dB = DevMatrix(b, K, N, N, 2, gap=np.nan)
        dC = DevMatrix(c, M, N, N, 3, gap=np.nan)
        st = sg.sgemm_general(cid, 0, 0, M, N, K, 1.0, dA.ptr, K, dB.ptr, N, 0.0, dC.ptr, N, None, 0,
                              torch.cuda.current_stream())
        torch.cuda.synchronize()
        flat = dC.fetch()
        assert st == 0, st
        out = dC.window(flat)
        ref, bound = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, c, N)
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (name, worst, idx, out[idx], ref[idx])


@pytest.mark.parametrize("opA,opB", OPS)
def test_fringe_columns_beside_whole_tiles(opA, opB):
    """M and K multiples of the tile and 4 or 8 columns over on 16-byte aligned rows: the tiles
    run the whole-tile kernel (no edge tests; the grid stops at column N - r, a multiple of BN)
    and the fringe workgroups the last columns. Every configuration and operand form, checked
    as above."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    for n, cid in enumerate(matrix_configs()):
        bm, bn, threads = tile_of(cid)
        bk = int(sg.describe(cid)["tile"].split("x")[2])
        r = (4, 8)[n % 2]
        steps = 2 if r == 4 else 1
        K = bk * max(1, min(4, 3 * threads * steps // bk))
        M, N = 2 * bm, 128 * bn + r
        st, grid, _ = sg.sgemm_launch_shape(cid, M, N, K)
        assert st == 0 and grid[0] == 256 + M // 2, (cid, grid)
        rng = np.random.default_rng(7 * cid + 100 * opA + 1000 * opB)
        a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
        bias = draw(rng, (N,), "normal") if n % 3 == 0 else None
        As, Bs = stored(opA, a), stored(opB, b)
        lda, ldb, ldc = As.shape[1] + 4, Bs.shape[1] + 8, N + 4
        say(f"fringe beside whole tiles: config {cid} op {opA}{opB} {M}x{N}x{K} r {r}")
        dA = DevMatrix(As, As.shape[0], As.shape[1], lda, 0, gap=np.nan)
        dB = DevMatrix(Bs, Bs.shape[0], Bs.shape[1], ldb, 0, gap=np.nan)
        dC = DevMatrix(c, M, N, ldc, 0, gap=np.nan)
        dbias = torch.from_numpy(bias).cuda() if bias is not None else None
        st = sg.sgemm_general(cid, opA, opB, M, N, K, 0.5, dA.ptr, lda, dB.ptr, ldb, 1.5, dC.ptr, ldc, dbias, 0,
                              torch.cuda.current_stream())
        torch.cuda.synchronize()
        flat = dC.fetch()
        assert st == 0, (cid, st)
        assert dA.unchanged() and dB.unchanged() and dC.outside_unchanged(flat), cid
        out = dC.window(flat)
        rows, cols = fringe_samples(rng, M, N, r)
        check_entries(out, opA, opB, M, N, K, 0.5, As, Bs, 1.5, c, bias, 0, rows, cols, cid)
