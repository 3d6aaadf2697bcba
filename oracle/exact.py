"""Exact rational brute force for tiny GEMMs (test infrastructure only).

Every fp32 value is a dyadic rational, so ``fractions.Fraction`` evaluates
alpha * A * B + beta * C with no rounding at all. Pure-Python loops: use it on
problems of a few thousand multiply-adds.

It follows the same definition as the C oracle (each entry is the dot product
of a row of A with a column of B; AutoMine++ #4, "Current algorithm"; the result
is alpha*acc + beta*C with C unread when beta is zero; "Micro_gemm_4x4", section
"Final C write (alpha, beta)"), but in exact arithmetic, so it can pin the fp64 oracle: on small-integer
inputs the two must agree exactly, and otherwise the oracle must sit within its
own fp64 summation error of this result.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = ["sgemm_exact"]


def sgemm_exact(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, opA=0, opB=0, bias=None):
    """Return the exact result as an M x N nested list of Fractions.

    opA/opB = 1 read the transposed operand (A stored K x M, B stored N x K); bias
    (length N, by column) is added after the scaled product.
    """
    a = np.asarray(A, dtype=np.float32).reshape(-1)
    b = np.asarray(B, dtype=np.float32).reshape(-1)
    bb = None if bias is None else np.asarray(bias, dtype=np.float32).reshape(-1)
    fa = Fraction(float(np.float32(alpha)))
    fb = Fraction(float(np.float32(beta)))
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = Fraction(0)
            if fa != 0:
                for k in range(K):
                    av = a[k * lda + i] if opA else a[i * lda + k]
                    bv = b[j * ldb + k] if opB else b[k * ldb + j]
                    s += Fraction(float(av)) * Fraction(float(bv))
            t = Fraction(0)
            if fb != 0:
                c = np.asarray(C, dtype=np.float32).reshape(-1)
                t = fb * Fraction(float(c[i * ldc + j]))
            bias_j = Fraction(0) if bb is None else Fraction(float(bb[j]))
            row.append(fa * s + t + bias_j)
        out.append(row)
    return out
