"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is elementwise. Random inputs must land within the oracle's
bound |c - ref| <= 4*max(K,1)*2^-24*(|alpha|*sum|a*b| + |beta*c|). Cases with an
exact answer (small integers, identity, permutation) must match it bitwise.
Every call also checks that A and B are untouched, and that C outside its
M x N window, in the ldc gap and in guard bands, is too.
"""

import numpy as np
import pytest

import oracle
from gpu_util import run_gemm, say, DevMatrix
from workloads import WORKLOADS, draw, gpt2_linear_set, make

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def configs():
    """Every data-parallel configuration (the stream-K ones need a workspace and have
    their own tests)."""
    import tiled_fp32_gemm_02_amd as sg
    return [i for i, n in enumerate(sg.configs()) if not n.startswith(("sk_", "sk16_"))]


def check_against_oracle(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out, checks, what):
    assert all(checks.values()), (what, checks)
    ref, bound = oracle.sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    ok, worst, idx = oracle.within_bound(out, ref, bound)
    assert ok, f"{what}: max |err|/bound = {worst} at {idx}: got {out[idx]}, oracle {ref[idx]}"
    return worst


# ------------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["sq256", "sq1024", "ragged"])
def test_workload_full(name):
    w = WORKLOADS[name]
    A, B, C = make(w)
    say(f"workload {name}: {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta}")
    st, out, checks = run_gemm(w.M, w.N, w.K, w.alpha, A, B, w.beta, C, lda=w.lda_, ldb=w.ldb_,
                               ldc=w.ldc_, c_fill=np.nan if C is None else None)
    assert st == 0
    check_against_oracle(w.M, w.N, w.K, w.alpha, A, w.lda_, B, w.ldb_, w.beta, C, w.ldc_, out, checks, name)


def test_workload_sq4096_full_epilogue():
    """The 4096^3 product with alpha=1.5, beta=0.5, on the configuration and launch
    the benchmark times (the default choice, one call on the current stream)."""
    w = WORKLOADS["sq4096"]
    A, B, C = make(w)
    say("workload sq4096: 4096^3 alpha=1.5 beta=0.5 (full oracle)")
    st, out, checks = run_gemm(w.M, w.N, w.K, w.alpha, A, B, w.beta, C)
    assert st == 0
    worst = check_against_oracle(w.M, w.N, w.K, w.alpha, A, w.K, B, w.N, w.beta, C, w.N, out, checks,
                                 "sq4096")
    say(f"sq4096 worst |err|/bound = {worst:.4f}")


@pytest.mark.parametrize("which", [0, 1, 2])
def test_workload_gpt2_linears(which):
    name, X, W = gpt2_linear_set()[which]
    M, K = X.shape
    N = W.shape[1]
    say(f"workload {name}: {M}x{N}x{K}")
    st, out, checks = run_gemm(M, N, K, 1.0, X, W, 0.0, None, c_fill=np.nan)
    assert st == 0
    check_against_oracle(M, N, K, 1.0, X, K, W, N, 0.0, None, N, out, checks, name)


# ------------------------------------------------------------------ every configuration

@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 270, 133), (129, 65, 1000), (1, 1, 1),
                                   (33, 517, 8)])
def test_every_config(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "uniform")
    for cid in configs():
        say(f"config {cid} {M}x{N}x{K}")
        st, out, checks = run_gemm(M, N, K, 1.25, A, B, -0.5, C, config=cid)
        assert st == 0
        check_against_oracle(M, N, K, 1.25, A, K, B, N, -0.5, C, N, out, checks, f"config {cid}")


# ------------------------------------------------------------------ exact answers

@pytest.mark.parametrize("M,N,K", [(37, 53, 29), (129, 131, 65), (256, 256, 256), (300, 520, 777)])
def test_small_integers_bitwise(M, N, K):
    rng = np.random.default_rng(5 + K)
    A, B, C = (draw(rng, s, "smallint") for s in [(M, K), (K, N), (M, N)])
    ref, _ = oracle.sgemm(M, N, K, 2.0, A, K, B, N, -1.0, C, N)   # every value an integer < 2^24
    for cid in configs():
        say(f"small integers config {cid} {M}x{N}x{K}")
        st, out, checks = run_gemm(M, N, K, 2.0, A, B, -1.0, C, config=cid)
        assert st == 0 and all(checks.values()), checks
        assert np.array_equal(out.astype(np.float64), ref), f"config {cid}"


def test_identity_and_permutation_bitwise():
    rng = np.random.default_rng(9)
    M, K = 301, 259
    A = draw(rng, (M, K), "normal")
    I = np.eye(K, dtype=np.float32)
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[perm, np.arange(K)] = 1
    for cid in configs():
        say(f"identity/permutation config {cid}")
        st, out, checks = run_gemm(M, K, K, 1.0, A, I, 0.0, None, config=cid, c_fill=np.nan)
        assert st == 0 and all(checks.values()) and np.array_equal(out, A)
        st, out, checks = run_gemm(M, K, K, 1.0, A, P, 0.0, None, config=cid, c_fill=np.nan)
        assert st == 0 and all(checks.values()) and np.array_equal(out, A[:, perm])


# ------------------------------------------------------------------ edges

EDGE_SIZES = [1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 257]


@pytest.mark.parametrize("K", [1, 3, 8, 17, 64, 129])
def test_edge_sweep_bitwise(K):
    """Ragged M and N around every tile size, small-integer data, exact answers."""
    rng = np.random.default_rng(100 + K)
    Mx, Nx = max(EDGE_SIZES), max(EDGE_SIZES)
    A_all, B_all = draw(rng, (Mx, K), "smallint"), draw(rng, (K, Nx), "smallint")
    for M in EDGE_SIZES[::2]:
        for N in EDGE_SIZES[1::2]:
            A = np.ascontiguousarray(A_all[:M])
            B = np.ascontiguousarray(B_all[:, :N])
            ref, _ = oracle.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, None, N)
            for cid in configs():
                st, out, checks = run_gemm(M, N, K, 1.0, A, B, 0.0, None, config=cid, c_fill=np.nan)
                assert st == 0 and all(checks.values()), (M, N, K, cid, checks)
                assert np.array_equal(out.astype(np.float64), ref), (M, N, K, cid)
    say(f"edge sweep K={K} done")


@pytest.mark.parametrize("offsets,ld_pad", [((0, 0, 0), (0, 0, 0)), ((1, 2, 3), (0, 0, 0)),
                                            ((0, 0, 0), (1, 5, 3)), ((3, 1, 2), (4, 8, 12)),
                                            ((0, 0, 0), (4, 8, 12))])
def test_alignment_and_leading_dimensions(offsets, ld_pad):
    """Unaligned bases and leading dimensions larger than the row (vector and scalar paths)."""
    rng = np.random.default_rng(31)
    M, N, K = 200, 296, 152
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    lda, ldb, ldc = K + ld_pad[0], N + ld_pad[1], N + ld_pad[2]
    for cid in configs():
        say(f"alignment offsets={offsets} ld_pad={ld_pad} config {cid}")
        st, out, checks = run_gemm(M, N, K, 0.75, A, B, 1.5, C, lda=lda, ldb=ldb, ldc=ldc,
                                   offsets=offsets, config=cid)
        assert st == 0
        check_against_oracle(M, N, K, 0.75, A, K, B, N, 1.5, C, N, out, checks, f"config {cid}")


@pytest.mark.parametrize("lda", [(1 << 20) - 4, (1 << 20) - 3, 1 << 20])
def test_long_rows_of_A(lda):
    """Row strides at the direct-copy limit: just below 2^20 floats the copies' byte offsets
    inside a 256-row tile reach 2^30 (16-byte copies for the aligned stride, 4-byte copies
    for the odd one); from 2^20 on the call takes the register-staged element-wise path.
    All must agree with the oracle, on the direct-copy configurations and the auto choice."""
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(37)
    M, N, K = 260, 36, 40
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    names = sg.configs()
    for cid in [-1] + [i for i, n in enumerate(names) if n.startswith(("mfma_", "mfma16_")) and n.endswith("d")]:
        say(f"long rows lda={lda} config {cid}")
        st, out, checks = run_gemm(M, N, K, 1.25, A, B, -0.5, C, lda=lda, config=cid)
        assert st == 0
        check_against_oracle(M, N, K, 1.25, A, K, B, N, -0.5, C, N, out, checks, f"lda {lda} config {cid}")


# ------------------------------------------------------------------ epilogue special cases

def test_beta_zero_ignores_nan_in_C():
    rng = np.random.default_rng(41)
    M, N, K = 130, 260, 70
    A, B = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    for cid in configs():
        st, out, checks = run_gemm(M, N, K, 1.0, A, B, 0.0, None, config=cid, c_fill=np.nan)
        assert st == 0 and np.all(np.isfinite(out))
        check_against_oracle(M, N, K, 1.0, A, K, B, N, 0.0, None, N, out, checks, f"config {cid}")


@pytest.mark.parametrize("alpha,K,beta", [(0.0, 50, 0.5), (1.0, 0, 0.5), (0.0, 50, 0.0), (2.0, 0, 0.0)])
def test_quick_return_scales_C(alpha, K, beta):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(43)
    M, N = 77, 301
    C = draw(rng, (M, N), "uniform")
    dC = DevMatrix(C, M, N, N + 3)
    say(f"quick return alpha={alpha} K={K} beta={beta}")
    # A and B are never read: pass NULL
    st = sg.sgemm(M, N, K, alpha, None, max(K, 1), None, N, beta, dC.ptr, N + 3)
    torch.cuda.synchronize()
    assert st == 0
    out = dC.window()
    assert dC.outside_unchanged()
    assert np.array_equal(out, (np.float32(beta) * C) if beta != 0 else np.zeros_like(C))


def test_empty_result_touches_nothing():
    import torch
    import tiled_fp32_gemm_02_amd as sg
    dC = DevMatrix(None, 4, 4, 4, fill=1.0)
    assert sg.sgemm(0, 4, 4, 1.0, None, 4, None, 4, 0.0, dC.ptr, 4) == 0
    assert sg.sgemm(4, 0, 4, 1.0, None, 4, None, 1, 0.0, dC.ptr, 4) == 0
    torch.cuda.synchronize()
    assert dC.unchanged()


def test_alpha_power_of_two_scales_exactly():
    rng = np.random.default_rng(47)
    M, N, K = 256, 512, 384
    A, B = draw(rng, (M, K), "uniform"), draw(rng, (K, N), "uniform")
    st, c1, _ = run_gemm(M, N, K, 1.0, A, B, 0.0, None, c_fill=np.nan)
    st, c8, _ = run_gemm(M, N, K, 8.0, A, B, 0.0, None, c_fill=np.nan)
    st, cm, _ = run_gemm(M, N, K, -0.25, A, B, 0.0, None, c_fill=np.nan)
    assert np.array_equal(c8, 8 * c1) and np.array_equal(cm, -0.25 * c1)


# ------------------------------------------------------------------ invariants

def test_deterministic():
    w = WORKLOADS["sq1024"]
    A, B, _ = make(w)
    outs = [run_gemm(w.M, w.N, w.K, 1.0, A, B, 0.0, None, c_fill=np.nan)[1] for _ in range(3)]
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


def test_zero_padding_invariance():
    """Zero-padding K, M and N to tile multiples leaves the original window bitwise equal
    (up to the sign of zero) for a fixed configuration."""
    rng = np.random.default_rng(53)
    M, N, K = 200, 300, 100
    A, B = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    Mp, Np, Kp = 256, 512, 128
    Ap = np.zeros((Mp, Kp), np.float32); Ap[:M, :K] = A
    Bp = np.zeros((Kp, Np), np.float32); Bp[:K, :N] = B
    for cid in configs():
        _, c0, _ = run_gemm(M, N, K, 1.0, A, B, 0.0, None, config=cid, c_fill=np.nan)
        _, c1, _ = run_gemm(Mp, Np, Kp, 1.0, Ap, Bp, 0.0, None, config=cid, c_fill=np.nan)
        assert np.array_equal(c0, c1[:M, :N]), f"config {cid}"


def test_non_default_stream():
    import torch
    rng = np.random.default_rng(59)
    M, N, K = 512, 512, 512
    A, B = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal")
    s = torch.cuda.Stream()
    st, out, checks = run_gemm(M, N, K, 1.0, A, B, 0.0, None, stream=s, c_fill=np.nan)
    assert st == 0
    check_against_oracle(M, N, K, 1.0, A, K, B, N, 0.0, None, N, out, checks, "side stream")


def test_tensor_form():
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(61)
    M, N, K = 100, 200, 300
    A, B, C = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal"), draw(rng, (M, N), "normal")
    big = torch.from_numpy(np.pad(C, ((0, 0), (0, 7)))).cuda()
    Ct = big[:, :N]                          # a view with row stride N + 7
    out = sg.gemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), Ct, alpha=2.0, beta=0.5)
    torch.cuda.synchronize()
    ref, bound = oracle.sgemm(M, N, K, 2.0, A, K, B, N, 0.5, C, N)
    assert out.data_ptr() == Ct.data_ptr()
    assert oracle.within_bound(out.cpu().numpy(), ref, bound)[0]
    assert np.array_equal(big[:, N:].cpu().numpy(), np.zeros((M, 7), np.float32))
    with pytest.raises(ValueError, match="Size error"):
        sg.gemm(torch.zeros(4, 3, device="cuda"), torch.zeros(4, 3, device="cuda"))


# ------------------------------------------------------------------ strided-batched form

@pytest.mark.parametrize("bsz,M,N,K", [(12, 64, 64, 64), (5, 100, 37, 53), (3, 1024, 1024, 64)])
def test_strided_batched(bsz, M, N, K):
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(67 + bsz)
    A = draw(rng, (bsz, M, K), "normal")
    B = draw(rng, (bsz, K, N), "normal")
    C = draw(rng, (bsz, M, N), "normal")
    say(f"batched {bsz}x{M}x{N}x{K}")
    Ct = torch.from_numpy(C).cuda()
    sg.gemm_batched(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), Ct, alpha=1.5, beta=-1.0)
    torch.cuda.synchronize()
    out = Ct.cpu().numpy()
    for b in range(bsz):
        ref, bound = oracle.sgemm(M, N, K, 1.5, A[b], K, B[b], N, -1.0, C[b], N)
        ok, worst, idx = oracle.within_bound(out[b], ref, bound)
        assert ok, (b, worst, idx)


def test_strided_batched_shared_operand():
    """strideB = 0: one B for every batch (e.g. a shared weight)."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(71)
    bsz, M, N, K = 4, 96, 160, 72
    A = draw(rng, (bsz, M, K), "normal")
    B = draw(rng, (K, N), "normal")
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.full((bsz, M, N), float("nan"), device="cuda")
    st = sg.sgemm_strided_batched(M, N, K, 1.0, dA, K, M * K, dB, N, 0, 0.0, dC, N, M * N, bsz)
    torch.cuda.synchronize()
    assert st == 0
    out = dC.cpu().numpy()
    for b in range(bsz):
        ref, bound = oracle.sgemm(M, N, K, 1.0, A[b], K, B, N, 0.0, None, N)
        assert oracle.within_bound(out[b], ref, bound)[0], b
