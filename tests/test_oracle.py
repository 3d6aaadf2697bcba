"""Pins for the CPU oracle (CPU only).

Each test compares the oracle with something other than itself: values worked
by hand (tests/golden), closed forms, numpy's float64 matmul (a library special
case of the same definition), an exact rational evaluation, and invariants.
The last group plants mistakes in calls to the oracle (a dropped term, a wrong
sign, a transposed operand, an ignored scalar) and checks that a pin catches
each one.
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
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals


def f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def run(M, N, K, alpha, A, lda, B, ldb, beta=0.0, C=None, ldc=None):
    return oracle.sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc if ldc else N)


# ---------------------------------------------------------------- hand-worked values

def test_textbook_golden():
    g = read_golden("textbook_2x3x2.txt")
    M, N, K = int(g["M"][0]), int(g["N"][0]), int(g["K"][0])
    A, B = f32(g["A"]), f32(g["B"])
    ref, _ = run(M, N, K, 1.0, A, K, B, N)
    assert ref.reshape(-1).tolist() == g["AB"]
    ref, _ = run(M, N, K, g["alpha"][0], A, K, B, N, g["beta"][0], f32(g["C"]), N)
    assert ref.reshape(-1).tolist() == g["result"]


def test_outer_product_golden():
    g = read_golden("outer_product_3x2x2.txt")
    M, N, K = int(g["M"][0]), int(g["N"][0]), int(g["K"][0])
    A, B = f32(g["A"]), f32(g["B"])
    ref, _ = run(M, N, K, 1.0, A, K, B, N)
    assert ref.reshape(-1).tolist() == g["AB"]
    # the golden outer products sum to the golden product
    assert (np.array(g["outer0"]) + np.array(g["outer1"])).tolist() == g["AB"]
    # and the oracle run with K = 1 on each column/row pair gives each outer product
    for k, key in enumerate(["outer0", "outer1"]):
        col = np.ascontiguousarray(A.reshape(M, K)[:, k])
        row = np.ascontiguousarray(B.reshape(K, N)[k, :])
        ref_k, _ = run(M, N, 1, 1.0, col, 1, row, N)
        assert ref_k.reshape(-1).tolist() == g[key]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 3), (33, 65, 17), (64, 40, 96)])
def test_identity_right_and_left(M, N, K):
    rng = np.random.default_rng(11)
    A = draw(rng, (M, K), "uniform")
    ref, bound = run(M, K, K, 1.0, A, K, f32(np.eye(K)), K)
    assert np.array_equal(ref, A.astype(np.float64))
    B = draw(rng, (K, N), "normal")
    ref, _ = run(K, N, K, 1.0, f32(np.eye(K)), K, B, N)
    assert np.array_equal(ref, B.astype(np.float64))


def test_permutation_permutes_columns():
    rng = np.random.default_rng(12)
    M, K = 19, 23
    A = draw(rng, (M, K), "normal")
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[perm, np.arange(K)] = 1.0          # column j of A*P is column perm[j] of A
    ref, _ = run(M, K, K, 1.0, A, K, f32(P), K)
    assert np.array_equal(ref, A[:, perm].astype(np.float64))


def test_rank1_constant_along_k():
    # a_ik = u_i, b_kj = v_j  =>  (AB)_ij = K * u_i * v_j exactly
    rng = np.random.default_rng(13)
    M, N, K = 9, 14, 4096
    u = rng.integers(-8, 9, size=M).astype(np.float32)
    v = rng.integers(-8, 9, size=N).astype(np.float32)
    A = f32(np.repeat(u[:, None], K, axis=1))
    B = f32(np.repeat(v[None, :], K, axis=0))
    ref, bound = run(M, N, K, 1.0, A, K, B, N)
    assert np.array_equal(ref, K * np.outer(u, v).astype(np.float64))
    assert np.array_equal(bound, 4 * K * U * K * np.abs(np.outer(u, v)).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(5, 7, 11), (16, 3, 64), (3, 16, 257)])
def test_sum_of_squares_closed_form(M, N, K):
    # a_ik = k, b_kj = k  =>  (AB)_ij = sum k^2 = (K-1) K (2K-1) / 6
    # (a transposed A gives i*K(K-1)/2 and a transposed B gives j*K(K-1)/2 instead)
    A = f32(np.tile(np.arange(K), (M, 1)))
    B = f32(np.tile(np.arange(K)[:, None], (1, N)))
    ref, _ = run(M, N, K, 1.0, A, K, B, N)
    assert np.all(ref == (K - 1) * K * (2 * K - 1) / 6)


def test_outer_of_indices_closed_form():
    # a_ik = i + 1, b_kj = j + 1  =>  (AB)_ij = K (i + 1)(j + 1): fixes where i and j land
    M, N, K = 6, 10, 13
    A = f32(np.tile(np.arange(1, M + 1)[:, None], (1, K)))
    B = f32(np.tile(np.arange(1, N + 1), (K, 1)))
    ref, _ = run(M, N, K, 1.0, A, K, B, N)
    i, j = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    assert np.array_equal(ref, K * (i + 1.0) * (j + 1.0))


@pytest.mark.parametrize("K", [1, 2, 7, 8, 100])
def test_alternating_signs(K):
    # a_ik = 1, b_kj = (-1)^k  =>  s = K mod 2, g = K
    A = f32(np.ones((3, K)))
    B = f32(np.tile(((-1.0) ** np.arange(K))[:, None], (1, 4)))
    ref, bound = run(3, 4, K, 1.0, A, K, B, 4)
    assert np.all(ref == K % 2)
    assert np.all(bound == 4 * K * U * K)


def test_bound_closed_form_ones():
    # A = B = 1, C = 1: g = K, t = beta, bound = 4 K u (|alpha| K + |beta|)
    M, N, K, alpha, beta = 4, 5, 9, -1.5, 0.25
    ref, bound = run(M, N, K, alpha, f32(np.ones((M, K))), K, f32(np.ones((K, N))), N,
                     beta, f32(np.ones((M, N))), N)
    assert np.all(ref == alpha * K + beta)
    assert np.all(bound == 4 * K * U * (abs(alpha) * K + abs(beta)))


def test_nonnegative_inputs_g_equals_s():
    rng = np.random.default_rng(14)
    M, N, K = 12, 9, 31
    A = f32(np.abs(draw(rng, (M, K), "normal")))
    B = f32(np.abs(draw(rng, (K, N), "normal")))
    ref, bound = run(M, N, K, 1.0, A, K, B, N)
    np.testing.assert_allclose(bound, 4 * K * U * ref, rtol=1e-15)


# ---------------------------------------------------------------- epilogue special cases

def test_beta_zero_never_reads_C():
    rng = np.random.default_rng(15)
    M, N, K = 8, 6, 5
    A, B = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    ref0, b0 = run(M, N, K, 2.0, A, K, B, N)
    Cnan = f32(np.full((M, N), np.nan))
    ref, b = run(M, N, K, 2.0, A, K, B, N, 0.0, Cnan, N)
    assert np.all(np.isfinite(ref)) and np.array_equal(ref, ref0) and np.array_equal(b, b0)


@pytest.mark.parametrize("alpha,K", [(0.0, 7), (1.0, 0), (0.0, 0)])
def test_alpha_zero_or_empty_k_is_beta_c(alpha, K):
    rng = np.random.default_rng(16)
    M, N = 5, 4
    A = f32(np.full((M, max(K, 1)), np.nan))   # must not be read
    B = f32(np.full((max(K, 1), N), np.nan))
    C = draw(rng, (M, N), "uniform")
    ref, bound = oracle.sgemm(M, N, K, alpha, A, max(K, 1), B, N, 0.75, C, N)
    t = 0.75 * C.astype(np.float64)
    assert np.array_equal(ref, t)
    assert np.array_equal(bound, 4 * max(K, 1) * U * np.abs(t))


def test_empty_result():
    ref, bound = oracle.sgemm(0, 5, 3, 1.0, None, 3, None, 5, 0.0, None, 5)
    assert ref.shape == (0, 5)
    ref, bound = oracle.sgemm(4, 0, 3, 1.0, None, 3, None, 1, 0.0, None, 1)
    assert ref.shape == (4, 0)


# ---------------------------------------------------------------- library and exact arithmetic

@pytest.mark.parametrize("M,N,K,alpha,beta", [(37, 53, 29, 1.0, 0.0), (64, 33, 130, -1.25, 0.5),
                                              (1, 300, 77, 3.0, -2.0), (129, 1, 64, 1.0, 1.0)])
def test_matches_numpy_float64(M, N, K, alpha, beta):
    rng = np.random.default_rng(17)
    lda, ldb, ldc = K + 3, N + 5, N + 1
    A = np.full((M, lda), np.nan, np.float32); A[:, :K] = draw(rng, (M, K), "normal")
    B = np.full((K, ldb), np.nan, np.float32); B[:, :N] = draw(rng, (K, N), "uniform")
    C = np.full((M, ldc), np.nan, np.float32); C[:, :N] = draw(rng, (M, N), "uniform")
    ref, bound = oracle.sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    a64, b64, c64 = (x.astype(np.float64) for x in (A[:, :K], B[:, :N], C[:, :N]))
    lib = alpha * (a64 @ b64) + beta * c64
    g = np.abs(a64) @ np.abs(b64)
    assert np.all(np.abs(ref - lib) <= 1e-12 * (abs(alpha) * g + abs(beta) * np.abs(c64)))
    np.testing.assert_allclose(bound, 4 * K * U * (abs(alpha) * g + np.abs(beta * c64)), rtol=1e-12)


def test_small_integers_exact():
    rng = np.random.default_rng(18)
    M, N, K = 7, 9, 13
    A, B, C = (draw(rng, s, "smallint") for s in [(M, K), (K, N), (M, N)])
    ref, _ = oracle.sgemm(M, N, K, 3.0, A, K, B, N, -2.0, C, N)
    exact = sgemm_exact(M, N, K, 3.0, A, K, B, N, -2.0, C, N)
    assert ref.tolist() == [[float(x) for x in row] for row in exact]


def test_within_fp64_error_of_exact():
    rng = np.random.default_rng(19)
    M, N, K = 4, 5, 40
    A, B = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    ref, bound = oracle.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, None, N)
    exact = sgemm_exact(M, N, K, 1.0, A, K, B, N, 0.0, None, N)
    g = bound / (4 * K * U)
    for i in range(M):
        for j in range(N):
            # fp64 summation of K exact products: error <= (K-1) * 2^-53 * g
            assert abs(ref[i, j] - float(exact[i][j])) <= (K - 1) * 2.0 ** -53 * g[i, j] * 1.0001


# ---------------------------------------------------------------- invariants and consistency

def test_ld_invariance():
    rng = np.random.default_rng(20)
    M, N, K = 21, 17, 19
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    r0, b0 = oracle.sgemm(M, N, K, 0.5, A, K, B, N, 2.0, C, N)
    Ap = np.full((M, K + 7), np.nan, np.float32); Ap[:, :K] = A
    Bp = np.full((K, N + 2), np.nan, np.float32); Bp[:, :N] = B
    Cp = np.full((M, N + 9), np.nan, np.float32); Cp[:, :N] = C
    r1, b1 = oracle.sgemm(M, N, K, 0.5, Ap, K + 7, Bp, N + 2, 2.0, Cp, N + 9)
    assert np.array_equal(r0, r1) and np.array_equal(b0, b1)


def test_entries_equal_full():
    rng = np.random.default_rng(21)
    M, N, K = 50, 70, 90
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    ref, bound = oracle.sgemm(M, N, K, 1.5, A, K, B, N, 0.5, C, N)
    rows = rng.integers(0, M, 300)
    cols = rng.integers(0, N, 300)
    r, b = oracle.sgemm_entries(M, N, K, 1.5, A, K, B, N, 0.5, C, N, rows, cols)
    assert np.array_equal(r, ref[rows, cols]) and np.array_equal(b, bound[rows, cols])
    with pytest.raises(IndexError):
        oracle.sgemm_entries(M, N, K, 1.5, A, K, B, N, 0.5, C, N, [M], [0])


def test_alpha_beta_linearity():
    """With small-integer A, B and C every result is exact in fp64, so the scalars and the
    operands must act linearly and exactly: alpha = 0, beta = 1 gives C; r(alpha, beta) =
    alpha * r(1, 0) + beta * C; and the product is additive in A and in B."""
    rng = np.random.default_rng(23)
    M, N, K = 11, 13, 17
    A1, A2 = draw(rng, (M, K), "smallint"), draw(rng, (M, K), "smallint")
    B1, B2 = draw(rng, (K, N), "smallint"), draw(rng, (K, N), "smallint")
    C = draw(rng, (M, N), "smallint")
    c64 = C.astype(np.float64)

    def r(alpha, A, B, beta):
        return oracle.sgemm(M, N, K, alpha, f32(A), K, f32(B), N, beta, C, N)[0]

    prod = r(1.0, A1, B1, 0.0)
    assert np.array_equal(r(0.0, A1, B1, 1.0), c64)
    for alpha, beta in [(3.0, -2.0), (-0.5, 0.25), (2.0, 1.0)]:
        assert np.array_equal(r(alpha, A1, B1, beta), alpha * prod + beta * c64)
    assert np.array_equal(r(1.0, A1 + A2, B1, 0.0), prod + r(1.0, A2, B1, 0.0))
    assert np.array_equal(r(1.0, A1, B1 + B2, 0.0), prod + r(1.0, A1, B2, 0.0))


def test_bound_admits_fp32_summation_orders():
    """Results a correct fp32 kernel may produce lie within the bound: forward,
    reverse, pairwise and 16-wide blocked sums, with and without fused multiply-add,
    with the epilogue rounded in fp32."""
    rng = np.random.default_rng(22)
    M, N, K = 6, 8, 1024
    A, B, C = draw(rng, (M, K), "uniform"), draw(rng, (K, N), "uniform"), draw(rng, (M, N), "uniform")
    alpha, beta = np.float32(1.5), np.float32(0.5)
    ref, bound = oracle.sgemm(M, N, K, float(alpha), A, K, B, N, float(beta), C, N)
    worst = 0.0
    for i in range(M):
        for j in range(N):
            p32 = (A[i, :] * B[:, j]).astype(np.float32)                 # rounded products
            pex = A[i, :].astype(np.float64) * B[:, j].astype(np.float64)  # fma: exact products
            cands = []
            for prods in (p32, pex):
                s = np.float32(0)
                for x in prods:                                 # forward
                    s = np.float32(np.float64(s) + x)
                cands.append(s)
                s = np.float32(0)
                for x in prods[::-1]:                           # reverse
                    s = np.float32(np.float64(s) + x)
                cands.append(s)
                blk = [np.float32(0)] * 16                      # 16 partial sums, then combined
                for k, x in enumerate(prods):
                    blk[k % 16] = np.float32(np.float64(blk[k % 16]) + x)
                s = np.float32(0)
                for x in blk:
                    s = np.float32(s + x)
                cands.append(s)
            cands.append(np.float32(np.sum(p32, dtype=np.float32)))  # numpy pairwise
            for s in cands:
                out = np.float32(np.float32(alpha * s) + np.float32(beta * C[i, j]))
                r = abs(float(out) - ref[i, j]) / bound[i, j]
                worst = max(worst, r)
    assert worst <= 1.0, worst


# ---------------------------------------------------------------- planted mistakes

def _pins_pass(call):
    """Run a small battery of pins against `call` (same signature as oracle.sgemm).
    Returns the list of pins that failed; a pin whose call raises has failed too."""
    failed = []

    def pin(name, check):
        try:
            ok = check()
        except (ValueError, IndexError, TypeError):
            ok = False
        if not ok:
            failed.append(name)

    def sum_of_squares():
        # non-square: catches transposed operands and dropped terms
        M, N, K = 5, 7, 11
        A = f32(np.tile(np.arange(K), (M, 1)))
        B = f32(np.tile(np.arange(K)[:, None], (1, N)))
        ref, _ = call(M, N, K, 1.0, A, K, B, N, 0.0, None, N)
        return ref.shape == (M, N) and bool(np.all(ref == (K - 1) * K * (2 * K - 1) / 6))

    def square_structured():
        # a_ik = k, b_kj = j + 1  =>  (AB)_ij = (j+1) K (K-1) / 2
        K = 9
        A = f32(np.tile(np.arange(K), (K, 1)))
        B = f32(np.tile(np.arange(1, K + 1), (K, 1)))
        ref, _ = call(K, K, K, 1.0, A, K, B, K, 0.0, None, K)
        jj = np.arange(1, K + 1)[None, :]
        return np.array_equal(ref, np.broadcast_to(jj * K * (K - 1) / 2.0, (K, K)))

    def golden_alpha_beta():
        g = read_golden("textbook_2x3x2.txt")
        ref, _ = call(2, 2, 3, g["alpha"][0], f32(g["A"]), 3, f32(g["B"]), 2, g["beta"][0], f32(g["C"]), 2)
        return ref.reshape(-1).tolist() == g["result"]

    def first_k():
        # a_i0 = 1, b_0j = j+1, every other term zero
        K = 6
        A = np.zeros((3, K), np.float32); A[:, 0] = 1
        B = np.zeros((K, 4), np.float32); B[0, :] = np.arange(1, 5)
        ref, _ = call(3, 4, K, 1.0, A, K, B, 4, 0.0, None, 4)
        return np.array_equal(ref, np.tile(np.arange(1.0, 5.0), (3, 1)))

    pin("sum_of_squares", sum_of_squares)
    pin("square_structured", square_structured)
    pin("golden_alpha_beta", golden_alpha_beta)
    pin("first_k", first_k)
    return failed


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.sgemm) == []


def _swap_index(X, rows, cols, ld):
    """Buffer whose (r, c) entry is read from X at c*ld + r: what an implementation
    that swaps the two indices of an operand would see (NaN where that falls
    outside the buffer)."""
    flat = np.asarray(X, np.float32).reshape(-1)
    out = np.full(max(rows, 1) * ld, np.nan, np.float32)
    for r in range(rows):
        for c in range(cols):
            idx = c * ld + r
            out[r * ld + c] = flat[idx] if idx < flat.size else np.nan
    return out


def _mut(fn):
    return lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: fn(M, N, K, al, A, lda, B, ldb, be, C, ldc)


MUTANTS = {
    "drop_last_k": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, max(K - 1, 0), al, A, lda, B, ldb, be, C, ldc)),
    "drop_first_k": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K - 1, al, np.asarray(A, np.float32).reshape(-1)[1:], lda,
        np.asarray(B, np.float32).reshape(-1)[ldb:], ldb, be, C, ldc)),
    "negated": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, -al, A, lda, B, ldb, be, C, ldc)),
    "ignores_alpha": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, 1.0, A, lda, B, ldb, be, C, ldc)),
    "alpha_beta_swapped": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, be, A, lda, B, ldb, al, C, ldc)),
    "ignores_beta": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, al, A, lda, B, ldb, 0.0, None, ldc)),
    "transposed_A": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, al, _swap_index(A, M, K, lda), lda, B, ldb, be, C, ldc)),
    "transposed_B": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: oracle.sgemm(
        M, N, K, al, A, lda, _swap_index(B, K, N, ldb), ldb, be, C, ldc)),
    "transposed_result": _mut(lambda M, N, K, al, A, lda, B, ldb, be, C, ldc: (
        lambda r: (r[0].T.copy() if M == N else np.full((M, N), np.nan), r[1]))(
        oracle.sgemm(M, N, K, al, A, lda, B, ldb, be, C, ldc))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    assert _pins_pass(MUTANTS[name]) != [], f"mutant {name} passed every pin"


# ---------------------------------------------------------------- the pass criterion

def test_within_bound_criterion():
    ref = np.array([1.0, -2.0, 0.0, 5.0])
    bound = np.array([0.5, 0.25, 0.0, 1.0])
    assert oracle.within_bound(np.float32([1.5, -2.25, 0.0, 4.0]), ref, bound)[0]   # at the edge
    ok, worst, idx = oracle.within_bound(np.float32([1.0, -2.0, 0.0, 6.5]), ref, bound)
    assert not ok and worst == 1.5 and idx == (3,)
    assert not oracle.within_bound(np.float32([1.0, -2.0, 1e-30, 5.0]), ref, bound)[0]  # zero bound
    assert not oracle.within_bound(np.float32([np.nan, -2.0, 0.0, 5.0]), ref, bound)[0]
    assert not oracle.within_bound(np.float32([np.inf, -2.0, 0.0, 5.0]), ref, bound)[0]
    assert oracle.within_bound(np.float32([1.0, -2.0, -0.0, 5.0]), ref, bound)[0]       # -0 == +0
