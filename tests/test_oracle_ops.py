"""Pins for the oracle's operand transposes, bias and GELU (CPU only).

Transposes: numpy float64 matmul of the transposed arrays (a library special case),
exact rational arithmetic, and a closed form whose value changes if either index
of a transposed read is swapped. Bias: a hand-worked golden and closed forms.
GELU (tanh form): torch's own tanh-form GELU in float64 (a library routine), the
exact erf-based GELU within the approximation's known error, the identity
gelu(x) - gelu(-x) = x, and the slope cap the error bound relies on.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle.exact import sgemm_exact
from workloads import draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24


def read_golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals


def stored(op, x, ld_pad=0):
    """The buffer an operand read as `x` is stored in under op (transposed if op), padded."""
    s = np.ascontiguousarray(x.T if op else x, dtype=np.float32)
    if ld_pad:
        s = np.ascontiguousarray(np.pad(s, ((0, 0), (0, ld_pad)), constant_values=np.nan))
    return s


@pytest.mark.parametrize("opA,opB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(37, 53, 29), (5, 70, 130), (64, 1, 9)])
def test_transposes_match_numpy(opA, opB, M, N, K):
    rng = np.random.default_rng(M + N + K + 10 * opA + 20 * opB)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    bias = draw(rng, (N,), "normal")
    As, Bs = stored(opA, a, 3), stored(opB, b, 5)
    ref, bound = oracle.gemm(opA, opB, M, N, K, -0.75, As, As.shape[1], Bs, Bs.shape[1], 1.25, c, N, bias)
    a64, b64, c64 = a.astype(np.float64), b.astype(np.float64), c.astype(np.float64)
    lib = -0.75 * (a64 @ b64) + 1.25 * c64 + bias.astype(np.float64)
    mag = 0.75 * (np.abs(a64) @ np.abs(b64)) + 1.25 * np.abs(c64) + np.abs(bias)
    assert np.all(np.abs(ref - lib) <= 1e-12 * mag)
    np.testing.assert_allclose(bound, 4 * (K + 1) * U * mag, rtol=1e-12)


@pytest.mark.parametrize("opA,opB", [(0, 1), (1, 0), (1, 1)])
def test_transposes_exact_small_integers(opA, opB):
    rng = np.random.default_rng(3 + opA + 2 * opB)
    M, N, K = 6, 7, 11
    a, b, c = (draw(rng, s, "smallint") for s in [(M, K), (K, N), (M, N)])
    bias = draw(rng, (N,), "smallint")
    As, Bs = stored(opA, a), stored(opB, b)
    ref, _ = oracle.gemm(opA, opB, M, N, K, 3.0, As, As.shape[1], Bs, Bs.shape[1], -1.0, c, N, bias)
    exact = sgemm_exact(M, N, K, 3.0, As, As.shape[1], Bs, Bs.shape[1], -1.0, c, N, opA=opA, opB=opB,
                        bias=bias)
    assert ref.tolist() == [[float(x) for x in row] for row in exact]


@pytest.mark.parametrize("opA,opB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_transposes_sum_of_squares(opA, opB):
    # a_ik = k and b_kj = k whatever the storage: (AB)_ij = (K-1) K (2K-1) / 6. Reading a
    # transposed operand with its indices swapped gives i*K(K-1)/2 or j*K(K-1)/2 instead.
    M, N, K = 5, 7, 11
    a = np.tile(np.arange(K, dtype=np.float32), (M, 1))
    b = np.tile(np.arange(K, dtype=np.float32)[:, None], (1, N))
    As, Bs = stored(opA, a), stored(opB, b)
    ref, _ = oracle.gemm(opA, opB, M, N, K, 1.0, As, As.shape[1], Bs, Bs.shape[1], 0.0, None, N)
    assert np.all(ref == (K - 1) * K * (2 * K - 1) / 6)


@pytest.mark.parametrize("opA,opB", [(0, 1), (1, 0), (1, 1)])
def test_forgotten_transpose_fails_the_closed_form(opA, opB):
    # planted mistake: a transposed operand read as if stored plainly (square, so it stays in range)
    K = M = N = 9
    a = np.tile(np.arange(K, dtype=np.float32), (M, 1))
    b = np.tile(np.arange(K, dtype=np.float32)[:, None], (1, N))
    As, Bs = stored(opA, a), stored(opB, b)
    bad, _ = oracle.gemm(0, 0, M, N, K, 1.0, As, K, Bs, N, 0.0, None, N)
    assert not np.all(bad == (K - 1) * K * (2 * K - 1) / 6)


def test_transposed_view_equals_plain():
    rng = np.random.default_rng(77)
    M, N, K = 33, 21, 45
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    r0, b0 = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N)
    r1, b1 = oracle.gemm(1, 1, M, N, K, 1.0, stored(1, a), M, stored(1, b), K, 0.0, None, N)
    assert np.array_equal(r0, r1) and np.array_equal(b0, b1)


def test_bias_golden():
    g = read_golden("bias_2x3x2.txt")
    A, B, bias = (np.float32(g[k]) for k in ("A", "B", "bias"))
    ref, _ = oracle.gemm(0, 0, 2, 2, 3, 1.0, A, 3, B, 2, 0.0, None, 2, bias)
    assert ref.reshape(-1).tolist() == g["AB_bias"]
    ref, _ = oracle.gemm(0, 0, 2, 2, 3, g["alpha"][0], A, 3, B, 2, g["beta"][0], np.float32(g["C"]), 2, bias)
    assert ref.reshape(-1).tolist() == g["result"]


@pytest.mark.parametrize("alpha,K", [(0.0, 5), (1.0, 0)])
def test_bias_on_quick_return(alpha, K):
    M, N = 3, 4
    c = np.arange(M * N, dtype=np.float32).reshape(M, N)
    bias = np.float32([1, -2, 3, -4])
    ref, bound = oracle.gemm(0, 0, M, N, K, alpha, None, max(K, 1), None, N, 0.5, c, N, bias)
    assert np.array_equal(ref, 0.5 * c + bias)
    assert np.array_equal(bound, 4 * (max(K, 1) + 1) * U * (np.abs(0.5 * c) + np.abs(bias)))


# ------------------------------------------------------------------ GELU

XS = np.concatenate([np.linspace(-12, 12, 4801), [-1e3, -30, 30, 1e3, 1e-8, -1e-8]])


def test_gelu_matches_torch_tanh_gelu():
    torch = pytest.importorskip("torch")
    x = torch.tensor(XS, dtype=torch.float64)
    lib = torch.nn.functional.gelu(x, approximate="tanh").numpy()
    ours = np.array([oracle.gelu_tanh(v) for v in XS])
    assert np.all(np.abs(ours - lib) <= 4e-16 * (np.abs(lib) + np.abs(XS) + 1e-300))


def test_gelu_close_to_exact_erf_gelu():
    # the tanh form approximates x * Phi(x); its largest gap is about 5e-4 (so the
    # pin fails for a wrong constant, a missing cube or the wrong branch of the formula)
    worst = max(abs(oracle.gelu_tanh(v) - 0.5 * v * (1 + math.erf(v / math.sqrt(2)))) for v in XS)
    assert 1e-5 < worst < 1e-3


def test_gelu_identities():
    for v in XS:
        assert abs((oracle.gelu_tanh(v) - oracle.gelu_tanh(-v)) - v) <= 4e-16 * max(abs(v), 1.0)
    assert oracle.gelu_tanh(0.0) == 0.0
    h = 1e-6
    assert abs((oracle.gelu_tanh(h) - oracle.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9
    assert oracle.gelu_tanh(30.0) == 30.0 and oracle.gelu_tanh(-30.0) == 0.0


def test_gelu_slope_cap():
    # the bound carries input error through the activation with factor 1.13
    x = np.linspace(-8, 8, 160001)
    g = np.array([oracle.gelu_tanh(v) for v in x])
    slope = np.abs(np.diff(g) / np.diff(x))
    assert 1.12 < slope.max() < 1.13


def test_gelu_fp32_evaluation_within_bound():
    # an fp32 evaluation of the same formula stays within 8 u (|t| + |gelu(t)|)
    t32 = np.float32(XS[:-6])
    c = np.float32(math.sqrt(2 / math.pi))
    inner = c * (t32 + np.float32(0.044715) * t32 * t32 * t32)
    g32 = np.float32(0.5) * t32 * (np.float32(1) + np.tanh(inner))
    ref = np.array([oracle.gelu_tanh(float(v)) for v in t32])
    err = np.abs(g32.astype(np.float64) - ref)
    assert np.all(err <= 8 * U * (np.abs(t32) + np.abs(ref)))


def test_gemm_with_gelu_applies_the_activation():
    rng = np.random.default_rng(5)
    M, N, K = 9, 12, 40
    a, b = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal002")
    bias = draw(rng, (N,), "normal")
    r0, b0 = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias, oracle.ACT_NONE)
    r1, b1 = oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias, oracle.ACT_GELU_TANH)
    assert np.array_equal(r1, np.vectorize(oracle.gelu_tanh)(r0))
    assert np.allclose(b1, 1.13 * b0 + 8 * U * (np.abs(r0) + np.abs(r1)), rtol=1e-14)
    with pytest.raises(ValueError):
        oracle.gemm(0, 0, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias, 2)


def test_entries_equal_full_with_ops():
    rng = np.random.default_rng(8)
    M, N, K = 40, 50, 60
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    bias = draw(rng, (N,), "normal")
    As, Bs = stored(1, a), stored(1, b)
    ref, bound = oracle.gemm(1, 1, M, N, K, 1.5, As, M, Bs, K, 0.5, c, N, bias, oracle.ACT_GELU_TANH)
    rows, cols = rng.integers(0, M, 200), rng.integers(0, N, 200)
    r, bd = oracle.gemm_entries(1, 1, M, N, K, 1.5, As, M, Bs, K, 0.5, c, N, rows, cols, bias,
                                oracle.ACT_GELU_TANH)
    assert np.array_equal(r, ref[rows, cols]) and np.array_equal(bd, bound[rows, cols])


# ------------------------------------------------------------------ planted mistakes

MUTANT_GELUS = {
    "erf_form": lambda x: 0.5 * x * (1 + math.erf(x / math.sqrt(2))),
    "coefficient": lambda x: 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.0447 * x ** 3))),
    "no_cube": lambda x: 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * x)),
    "no_half": lambda x: x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3))),
}


@pytest.mark.parametrize("name", sorted(MUTANT_GELUS))
def test_gelu_pin_catches_mutants(name):
    torch = pytest.importorskip("torch")
    x = torch.tensor(XS[:-6], dtype=torch.float64)
    lib = torch.nn.functional.gelu(x, approximate="tanh").numpy()
    mut = np.array([MUTANT_GELUS[name](v) for v in XS[:-6]])
    assert not np.all(np.abs(mut - lib) <= 4e-16 * (np.abs(lib) + np.abs(XS[:-6]) + 1e-300))
