"""Helpers for the GPU parity tests: device buffers with guard bands, one call
through the C ABI, and the checks that nothing outside the result was written."""

from __future__ import annotations

import sys

import numpy as np

CANARY = np.float32(-7.0e30)   # a value no tested product produces
GUARD = 64                     # floats of guard band before and after each buffer


def say(msg: str) -> None:
    """Name the case before a GPU step, so a failing run shows what it was doing."""
    print(msg, flush=True)
    sys.stdout.flush()


class DevMatrix:
    """A rows x ld float32 matrix inside a flat device buffer with guard bands.

    `offset` shifts the start by that many floats (0..3) to test unaligned bases.
    Columns >= `cols` (the ld gap) and the guard bands hold `gap` (CANARY by default).
    """

    def __init__(self, host: np.ndarray | None, rows: int, cols: int, ld: int, offset: int = 0,
                 fill=None, gap=CANARY):
        import torch
        self.rows, self.cols, self.ld, self.offset = rows, cols, ld, offset
        n = rows * ld
        self.flat = np.full(GUARD + offset + n + GUARD, gap, dtype=np.float32)
        win = self.flat[GUARD + offset: GUARD + offset + n].reshape(rows, ld) if n else None
        if n:
            if host is not None:
                win[:, :cols] = np.asarray(host, dtype=np.float32).reshape(rows, -1)[:, :cols]
            elif fill is not None:
                win[:, :cols] = fill
        self.dev = torch.from_numpy(self.flat.copy()).cuda()

    @property
    def ptr(self) -> int:
        return int(self.dev.data_ptr()) + 4 * (GUARD + self.offset)

    def fetch(self) -> np.ndarray:
        return self.dev.cpu().numpy()

    def window(self, flat: np.ndarray | None = None) -> np.ndarray:
        flat = self.fetch() if flat is None else flat
        n = self.rows * self.ld
        return flat[GUARD + self.offset: GUARD + self.offset + n].reshape(self.rows, self.ld)[:, :self.cols]

    def outside_unchanged(self, flat: np.ndarray | None = None) -> bool:
        """Everything but the rows x cols window is bit-identical to before."""
        flat = self.fetch() if flat is None else flat
        mask = np.ones(self.flat.size, dtype=bool)
        n = self.rows * self.ld
        if n:
            idx = np.arange(n).reshape(self.rows, self.ld)[:, :self.cols] + GUARD + self.offset
            mask[idx.reshape(-1)] = False
        return np.array_equal(flat[mask].view(np.uint32), self.flat[mask].view(np.uint32))

    def unchanged(self) -> bool:
        return np.array_equal(self.fetch().view(np.uint32), self.flat.view(np.uint32))


def run_gemm(M, N, K, alpha, A, B, beta, C, *, lda=None, ldb=None, ldc=None, offsets=(0, 0, 0),
             config=-1, stream=None, c_fill=None):
    """Run one product through sgemm_ex on freshly guarded device buffers.

    Returns (status, C window as float32 numpy array, checks) where checks is a dict of
    booleans: A and B untouched, C outside its window untouched.
    """
    import torch
    import tiled_fp32_gemm_02_amd as sg
    lda = lda or max(1, K)
    ldb = ldb or max(1, N)
    ldc = ldc or max(1, N)
    dA = DevMatrix(A, M, K, lda, offsets[0])
    dB = DevMatrix(B, K, N, ldb, offsets[1])
    dC = DevMatrix(C, M, N, ldc, offsets[2], fill=c_fill)
    s = stream if stream is not None else torch.cuda.current_stream()
    st = sg.sgemm_ex(config, M, N, K, alpha, dA.ptr, lda, dB.ptr, ldb, beta, dC.ptr, ldc, s)
    torch.cuda.synchronize()
    cflat = dC.fetch()
    checks = {"A_untouched": dA.unchanged(), "B_untouched": dB.unchanged(),
              "C_outside_untouched": dC.outside_unchanged(cflat)}
    return st, dC.window(cflat), checks
