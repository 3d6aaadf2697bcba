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


def sgemm_exact(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    """Return the exact result as an M x N nested list of Fractions."""
    a = np.asarray(A, dtype=np.float32).reshape(-1)
    b = np.asarray(B, dtype=np.float32).reshape(-1)
    fa = Fraction(float(np.float32(alpha)))
    fb = Fraction(float(np.float32(beta)))
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = Fraction(0)
            if fa != 0:
                for k in range(K):
                    s += Fraction(float(a[i * lda + k])) * Fraction(float(b[k * ldb + j]))
            t = Fraction(0)
            if fb != 0:
                c = np.asarray(C, dtype=np.float32).reshape(-1)
                t = fb * Fraction(float(c[i * ldc + j]))
            row.append(fa * s + t)
        out.append(row)
    return out
