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
* ``prob1024``: ``rng.random(shape, float32) * 2**-9``: non-negative entries whose
  rows of 1024 sum to about 1, standing in for attention probabilities after the
  softmax (exact in fp32: a power-of-two scale of multiples of 2**-24).

Draw order within one workload is A, then B, then C (C only when beta != 0).
The GPT-2-small linear set draws X1, W1, W2, X3, W3 from one generator; X1
feeds both the QKV and the MLP-up products.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Gemm", "WORKLOADS", "draw", "make", "gpt2_linear_set", "flops", "BatchedGemm", "gpt2_attention_set",
           "ATTENTION"]


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
    elif dist == "prob1024":
        x = rng.random(shape, dtype=np.float32) * np.float32(2.0 ** -9)
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


@dataclass(frozen=True)
class BatchedGemm:
    """One strided-batched product over shared buffers: for b in [0, batch),
    C_b = alpha * op(A_b) op(B_b) with A_b at float offset a_off + b*sA of buffer `a`
    (leading dimension lda), likewise B_b and C_b. op = 1 reads the stored matrix
    transposed. Names the buffers of ``gpt2_attention_set``."""

    name: str
    batch: int
    M: int
    N: int
    K: int
    alpha: float
    opA: int
    opB: int
    a: str
    a_off: int
    lda: int
    sA: int
    b: str
    b_off: int
    ldb: int
    sB: int
    c_rows: int
    c_cols: int
    c_off: int
    ldc: int
    sC: int
    note: str = field(default="", compare=False)


def gpt2_attention_set(seed: int = 5, T: int = 1024, heads: int = 12, hd: int = 64):
    """Inputs of one GPT-2-small attention layer's two per-head products at batch 1 x T
    tokens: the QKV projection output X[T x 3*heads*hd] ~ N(0, 1) (Q, K, V are its three
    column blocks, head h at columns h*hd of each) and probabilities P[heads x T x T]
    (``prob1024``), drawn in that order from one generator. P is drawn, not computed from
    the scores, so that each product's inputs are independent of the other's result."""
    rng = np.random.default_rng(seed)
    qkv = draw(rng, (T, 3 * heads * hd), "normal")
    p = draw(rng, (heads, T, T), "prob1024")
    return {"qkv": qkv, "p": p}


def attention_products(T: int = 1024, heads: int = 12, hd: int = 64):
    """The two batched products of attention over ``gpt2_attention_set`` buffers:
    scores_h = Q_h K_h^T / sqrt(hd) into S[heads x T x T], and out_h = P_h V_h written
    side by side into O[T x heads*hd] (head h at columns h*hd)."""
    w = 3 * heads * hd
    return [
        BatchedGemm("gpt2_attn_scores", heads, T, T, hd, 1.0 / float(np.sqrt(hd)), 0, 1,
                    "qkv", 0, w, hd, "qkv", heads * hd, w, hd, heads * T, T, 0, T, T * T,
                    note=f"{heads} heads x Q_h K_h^T / sqrt({hd}): {T}x{T}x{hd}, Q and K read in place from "
                         f"QKV[{T}x{w}] (K transposed)"),
        BatchedGemm("gpt2_attn_values", heads, T, hd, T, 1.0, 0, 0,
                    "p", 0, T, T * T, "qkv", 2 * heads * hd, w, hd, T, heads * hd, 0, heads * hd, hd,
                    note=f"{heads} heads x P_h V_h: {T}x{hd}x{T}, V read in place from QKV, heads side by side "
                         f"in O[{T}x{heads * hd}]"),
    ]


ATTENTION = {b.name: b for b in attention_products()}
