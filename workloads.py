"""Seeded synthetic inputs for the fp32 GEMM workloads.

This module only draws numbers. It holds none of the GEMM arithmetic, so both
sides of every comparison can use it: the HIP path (through the package binding)
and the CPU oracle under ``oracle/``.

The pages measure their kernels on unnamed or model-driven matrices (the SYCL
posts time an unstated square size against NumPy/MKL; the GPT-2 post runs a
trained model). No dataset is used here. Every matrix is drawn from
``numpy.random.default_rng(seed)`` (PCG64) in a fixed order, C-contiguous,
row-major, float32:

* ``uniform``: ``rng.random(shape, float32) * 2 - 1``. ``rng.random`` returns
  multiples of 2**-24 in [0, 1), so the affine map is exact in fp32 and lands
  in [-1, 1).
* ``normal``: ``rng.standard_normal(shape, float32)``.
* ``normal002``: ``0.02 * rng.standard_normal(shape, float32)`` (the usual
  init scale of a GPT-2 linear weight).

Draw order within one workload is A, then B, then C (C only when beta != 0).
The GPT-2-small linear set draws X1, W1, W2, X3, W3 from one generator; X1
feeds both the QKV and the MLP-up products.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Gemm", "WORKLOADS", "draw", "make", "gpt2_linear_set", "flops"]


@dataclass(frozen=True)
class Gemm:
    """One GEMM problem: sizes, leading dimensions, scalars and how inputs are drawn."""

    name: str
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    dist_a: str = "uniform"
    dist_b: str = "uniform"
    dist_c: str = "uniform"
    seed: int = 0
    lda: int | None = None
    ldb: int | None = None
    ldc: int | None = None
    note: str = field(default="", compare=False)

    @property
    def lda_(self) -> int:
        return self.lda if self.lda is not None else max(1, self.K)

    @property
    def ldb_(self) -> int:
        return self.ldb if self.ldb is not None else max(1, self.N)

    @property
    def ldc_(self) -> int:
        return self.ldc if self.ldc is not None else max(1, self.N)


def flops(M: int, N: int, K: int) -> int:
    """Algorithmic work of one GEMM: one multiply and one add per (i, j, k)."""
    return 2 * M * N * K


def draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """Draw one float32 matrix of ``shape`` from ``dist`` (see module docstring)."""
    if dist == "uniform":
        x = rng.random(shape, dtype=np.float32) * np.float32(2) - np.float32(1)
    elif dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "normal002":
        x = np.float32(0.02) * rng.standard_normal(shape, dtype=np.float32)
    elif dist == "smallint":
        # integers in [-8, 8]: every partial sum of K <= 2**17 products stays exact in fp32
        x = rng.integers(-8, 9, size=shape).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(x, dtype=np.float32)


def make(w: Gemm):
    """Draw (A, B, C) for workload ``w`` as row-major float32 arrays with their
    leading dimensions as the row length (A is M x lda, B is K x ldb, C is M x ldc).

    C is drawn only when beta != 0; otherwise it is None (the product ignores it).
    Entries in the padding columns (index >= K, N, N) are NaN so that any read
    of them shows up in a result. The GPT-2 workloads come from ``gpt2_linear_set``.
    """
    if w.name.startswith("gpt2_"):
        X, W = {name: (x, wt) for name, x, wt in gpt2_linear_set(w.seed)}[w.name]
        return X, W, None
    rng = np.random.default_rng(w.seed)
    A = _padded(draw(rng, (w.M, w.K), w.dist_a), w.lda_)
    B = _padded(draw(rng, (w.K, w.N), w.dist_b), w.ldb_)
    C = None
    if w.beta != 0.0:
        C = _padded(draw(rng, (w.M, w.N), w.dist_c), w.ldc_)
    return A, B, C


def _padded(x: np.ndarray, ld: int) -> np.ndarray:
    rows, cols = x.shape
    if ld == cols:
        return x
    out = np.full((rows, ld), np.nan, dtype=np.float32)
    out[:, :cols] = x
    return out


def gpt2_linear_set(seed: int = 4):
    """The three GPT-2-small linear layers at batch 1 x 1024 tokens.

    Returns ``[(name, X, W)]`` for QKV (768 -> 2304), MLP-up (768 -> 3072) and
    MLP-down (3072 -> 768). X ~ N(0, 1), W ~ N(0, 0.02**2), drawn in the order
    X1, W1, W2, X3, W3 from one generator; X1 feeds both of the first two.
    """
    rng = np.random.default_rng(seed)
    X1 = draw(rng, (1024, 768), "normal")
    W1 = draw(rng, (768, 2304), "normal002")
    W2 = draw(rng, (768, 3072), "normal002")
    X3 = draw(rng, (1024, 3072), "normal")
    W3 = draw(rng, (3072, 768), "normal002")
    return [("gpt2_qkv", X1, W1), ("gpt2_mlp_up", X1, W2), ("gpt2_mlp_down", X3, W3)]


WORKLOADS = {
    "sq256": Gemm("sq256", 256, 256, 256, seed=0,
                  note="256^3, U[-1,1), alpha=1, beta=0"),
    "sq1024": Gemm("sq1024", 1024, 1024, 1024, seed=1,
                   note="1024^3, U[-1,1), alpha=1, beta=0"),
    "sq4096": Gemm("sq4096", 4096, 4096, 4096, alpha=1.5, beta=0.5, seed=2,
                   note="4096^3, A,B,C U[-1,1), alpha=1.5, beta=0.5 (full epilogue)"),
    "ragged": Gemm("ragged", 1000, 1537, 777, dist_a="normal", dist_b="normal", seed=3,
                   note="1000x1537x777, N(0,1), lda=777, ldb=ldc=1537 (unaligned rows)"),
    "gpt2_qkv": Gemm("gpt2_qkv", 1024, 2304, 768, dist_a="normal", dist_b="normal002", seed=4,
                     note="GPT-2-small QKV projection, 1024 tokens: X[1024x768] W[768x2304]"),
    "gpt2_mlp_up": Gemm("gpt2_mlp_up", 1024, 3072, 768, dist_a="normal", dist_b="normal002", seed=4,
                        note="GPT-2-small MLP up, 1024 tokens: X[1024x768] W[768x3072]"),
    "gpt2_mlp_down": Gemm("gpt2_mlp_down", 1024, 768, 3072, dist_a="normal", dist_b="normal002", seed=4,
                          note="GPT-2-small MLP down, 1024 tokens: X[1024x3072] W[3072x768]"),
}
