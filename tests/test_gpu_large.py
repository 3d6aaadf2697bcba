"""GPU parity with operands that reach more than 2^31 floats past their base pointer.

Each case puts one operand in a device buffer of about 8.8 GB: its leading dimension
(just below or just above 2^20 floats, or 2^20 - 3) times its 2100 stored rows passes
2^31 floats, so the loaders' and the epilogue's offsets only fit in 64 bits. The buffer
is NaN-filled and only the used window holds data. A read outside the window turns
results into NaN, and a write outside C's window shows up in the columns checked next to
it. The cases cover A, B and C, plain and transposed, the direct-copy and the
register-staged loaders (a leading dimension of 2^20 and above takes the second), the
16x16 and vector-ALU kernels and a stream-K configuration. A last case is one compact
product of 2^22 + 1061 rows whose A alone holds more than 2^31 floats. Results are checked
against the oracle's bound.
"""

import numpy as np
import pytest

import oracle
from gpu_util import say
from workloads import draw

pytestmark = pytest.mark.gpu

BIG_ROWS = 2100
LDS = [(1 << 20) - 4, (1 << 20) - 3, (1 << 20) + 4]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def configs_to_run():
    """The automatic choice plus one configuration of every kernel family."""
    import tiled_fp32_gemm_02_amd as sg
    names = sg.configs()
    return [-1] + [names.index(n) for n in ("tile16", "valu_128x128x8_t8x8", "mfma_128x128x32_w2x2k2",
                                            "mfma_256x256x32_w2x4d", "sk_64x128x32_w2x2k2p2")]


class Placed:
    """A rows x cols host matrix at the top-left of a NaN-filled rows x ld device buffer."""

    def __init__(self, host, ld):
        import torch
        self.rows, self.cols = host.shape
        self.ld = ld
        self.buf = torch.full((self.rows * ld,), float("nan"), dtype=torch.float32, device="cuda")
        self.view = self.buf.view(self.rows, ld)
        self.view[:, :self.cols].copy_(torch.from_numpy(np.ascontiguousarray(host)))

    @property
    def ptr(self):
        return int(self.buf.data_ptr())

    def window(self):
        return self.view[:, :self.cols].cpu().numpy()

    def beside_window_untouched(self):
        """The 64 columns after the window, in every row, still hold the fill."""
        import torch
        hi = min(self.ld, self.cols + 64)
        return bool(torch.isnan(self.view[:, self.cols:hi]).all().item())


def run(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    ws = sg.workspace_for(torch.device("cuda"))
    st = sg.sgemm_general_ws(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None,
                             sg.SGEMM_ACT_NONE, ws, ws.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    return st


CASES = [
    # (name, opA, opB, M, N, K, which operand is the big one)
    ("A rows", 0, 0, BIG_ROWS, 64, 64, "A"),
    ("A transposed", 1, 0, 64, 64, BIG_ROWS, "A"),
    ("B rows", 0, 0, 64, 64, BIG_ROWS, "B"),
    ("B transposed", 0, 1, 64, BIG_ROWS, 64, "B"),
    ("C rows", 0, 0, BIG_ROWS, 64, 64, "C"),
]


@pytest.mark.parametrize("ld", LDS)
@pytest.mark.parametrize("name,opA,opB,M,N,K,big", CASES)
def test_offsets_past_2_31(name, opA, opB, M, N, K, big, ld):
    import torch
    rng = np.random.default_rng(M + 3 * N + 7 * K + opA + 2 * opB + ld % 97)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    As = np.ascontiguousarray(a.T if opA else a)
    Bs = np.ascontiguousarray(b.T if opB else b)
    alpha, beta = 1.25, (0.5 if big == "C" else 0.0)
    ref, bound = oracle.gemm(opA, opB, M, N, K, alpha, As, As.shape[1], Bs, Bs.shape[1], beta, c, N)
    lda = ld if big == "A" else As.shape[1]
    ldb = ld if big == "B" else Bs.shape[1]
    ldc = ld if big == "C" else N
    dA, dB = Placed(As, lda), Placed(Bs, ldb)
    for cid in configs_to_run():
        dC = Placed(c, ldc)
        say(f"large offsets: {name} {M}x{N}x{K} op {opA}{opB} ld {ld} config {cid}")
        st = run(cid, opA, opB, M, N, K, alpha, dA.ptr, lda, dB.ptr, ldb, beta, dC.ptr, ldc)
        assert st == 0, (name, cid, st)
        out = dC.window()
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (name, ld, cid, worst, idx, out[idx], ref[idx])
        assert dC.beside_window_untouched(), (name, ld, cid)
        del dC
    del dA, dB
    torch.cuda.empty_cache()


def test_more_than_2_31_floats_in_A():
    """A compact (2^22 + 1061) x 512 A: its last rows start past 2^31 floats. Rows are drawn
    from a block of 4093 random rows (row i is block row i % 4093), so the oracle checks
    sampled output rows from that block; with a prime period, a byte offset truncated to
    32 bits would land on a different block row."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    M, N, K, P = (1 << 22) + 1061, 64, 512, 4093
    rng = np.random.default_rng(2031)
    block, b = draw(rng, (P, K), "normal"), draw(rng, (K, N), "normal")
    dblock = torch.from_numpy(block).cuda()
    dA = dblock.repeat((M + P - 1) // P, 1)[:M]
    assert dA.is_contiguous() and dA.numel() > (1 << 31)
    dB = torch.from_numpy(b).cuda()
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    edge = (1 << 31) // K                              # first row whose offset reaches 2^31 floats
    assert edge + 64 <= M
    rows = np.unique(np.concatenate([np.arange(64), np.arange(edge - 64, edge + 64), np.arange(M - 64, M),
                                     np.random.default_rng(5).integers(0, M, 256)]))
    assert rows.min() >= 0 and rows.max() < M          # gathered from dC below
    ref, bound = oracle.gemm(0, 0, rows.size, N, K, 1.0, np.ascontiguousarray(block[rows % P]), K, b, N, 0.0,
                             None, N)
    for cid in [-1, sg.configs().index("mfma_128x128x32_w2x2k2")]:
        say(f"large A: {M}x{N}x{K} config {cid}")
        dC.fill_(float("nan"))
        st = sg.sgemm_general(cid, 0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dC.data_ptr(), N,
                              None, sg.SGEMM_ACT_NONE, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert st == 0
        out = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (cid, worst, idx, rows[idx[0]])
        assert not bool(torch.isnan(dC).any().item())      # every row written
    del dA, dB, dC, dblock
    torch.cuda.empty_cache()
