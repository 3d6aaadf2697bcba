"""GPU parity of the strided-batched products with operand forms (C ABI).

The GPT-2 post runs attention's per-head products through the batched variant of its
tiled kernel, on strided and transposed views without copies ("GPU Target - GPT-2 on
the GPU", section "Tiled matrix multiplication"). Here: the GPT-2-small shapes (12 heads,
1024 tokens, head size 64) with Q, K and V read in place from one QKV matrix and the
heads' outputs written side by side, a ragged head count and sequence length, every
kernel configuration in every operand form on a small batched problem, the exact
small-integer case, and bias + GELU. Every entry of every batch is checked against the
oracle, run per batch on the same buffer views; A, B and C outside its windows must be
untouched.
"""

import numpy as np
import pytest

import oracle
from gpu_util import say
from workloads import attention_products, draw, gpt2_attention_set

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def run_batched(prob, bufs, config=-1, bias=None, act=0, c_init=None):
    """Run one BatchedGemm on device copies of `bufs`; returns (status, C buffer after,
    C buffer before, {name: unchanged})."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    dev = {k: torch.from_numpy(np.ascontiguousarray(v).reshape(-1).copy()).cuda() for k, v in bufs.items()}
    c_before = (np.full(prob.c_rows * prob.c_cols, np.float32(-7.0e30), np.float32) if c_init is None
                else np.ascontiguousarray(c_init, np.float32).reshape(-1).copy())
    dC = torch.from_numpy(c_before.copy()).cuda()
    dbias = torch.from_numpy(bias).cuda() if bias is not None else None
    st = sg.sgemm_strided_batched_general(
        config, prob.opA, prob.opB, prob.M, prob.N, prob.K, prob.alpha,
        dev[prob.a].data_ptr() + 4 * prob.a_off, prob.lda, prob.sA,
        dev[prob.b].data_ptr() + 4 * prob.b_off, prob.ldb, prob.sB,
        0.0 if c_init is None else 0.5, dC.data_ptr() + 4 * prob.c_off, prob.ldc, prob.sC, dbias, act, prob.batch,
        torch.cuda.current_stream())
    torch.cuda.synchronize()
    unchanged = {k: np.array_equal(dev[k].cpu().numpy().view(np.uint32),
                                   np.ascontiguousarray(v).reshape(-1).view(np.uint32)) for k, v in bufs.items()}
    return st, dC.cpu().numpy(), c_before, unchanged


def check_batches(prob, bufs, out, c_before, bias=None, act=0, beta=0.0):
    """Every batch's window against the oracle; everything outside the windows unchanged."""
    written = np.zeros(out.size, bool)
    worst_all = 0.0
    for b in range(prob.batch):
        a = np.ascontiguousarray(bufs[prob.a]).reshape(-1)[prob.a_off + b * prob.sA:]
        bb = np.ascontiguousarray(bufs[prob.b]).reshape(-1)[prob.b_off + b * prob.sB:]
        c0 = c_before[prob.c_off + b * prob.sC:]
        ref, bound = oracle.gemm(prob.opA, prob.opB, prob.M, prob.N, prob.K, prob.alpha, a, prob.lda, bb, prob.ldb,
                                 beta, c0 if beta != 0.0 else None, prob.ldc, bias, act)
        idx = prob.c_off + b * prob.sC + np.arange(prob.M)[:, None] * prob.ldc + np.arange(prob.N)[None, :]
        ok, worst, where = oracle.within_bound(out[idx], ref, bound)
        assert ok, (prob.name, b, worst, where)
        assert not written[idx].any(), "batches wrote overlapping entries"
        written[idx] = True
        worst_all = max(worst_all, worst)
    assert np.array_equal(out[~written].view(np.uint32), c_before[~written].view(np.uint32)), \
        "entries outside the batches' windows were written"
    return worst_all


@pytest.mark.parametrize("name", ["gpt2_attn_scores", "gpt2_attn_values"])
def test_gpt2_attention_heads(name):
    """12 heads x 1024 tokens, head size 64: Q K^T / 8 with K transposed in place, and P V
    with the heads written side by side into one 1024 x 768 matrix."""
    prob = {p.name: p for p in attention_products()}[name]
    bufs = gpt2_attention_set()
    say(f"batched attention {name}: {prob.batch} x {prob.M}x{prob.N}x{prob.K}")
    st, out, c0, unchanged = run_batched(prob, bufs)
    assert st == 0 and all(unchanged.values()), (st, unchanged)
    check_batches(prob, bufs, out, c0)


@pytest.mark.parametrize("T,heads,hd", [(1000, 7, 64), (77, 5, 33), (130, 3, 40)])
def test_ragged_attention_heads(T, heads, hd):
    """A ragged head count and sequence length; head size 33 makes every row start only
    4-byte aligned (the 32-bit path)."""
    bufs = gpt2_attention_set(seed=T + heads, T=T, heads=heads, hd=hd)
    for prob in attention_products(T=T, heads=heads, hd=hd):
        say(f"batched attention {prob.name}: {heads} x {prob.M}x{prob.N}x{prob.K}")
        st, out, c0, unchanged = run_batched(prob, bufs)
        assert st == 0 and all(unchanged.values()), (st, unchanged)
        check_batches(prob, bufs, out, c0)


def small_problem(opA, opB, batch=3, M=100, N=70, K=50, pad=3, aligned=False):
    """A batched problem whose matrices sit inside shared buffers with padded rows, read in
    the given operand forms. Unaligned: buffer offsets of 1..3 floats and odd strides (the
    32-bit path). Aligned: sizes, leading dimensions and strides multiples of 4 and no
    offsets (the 128-bit path)."""
    from workloads import BatchedGemm
    if aligned:
        M, N, K, pad = (-(-x // 4) * 4 for x in (M, N, K, pad))
    ar, ac = (K, M) if opA else (M, K)
    br, bc = (N, K) if opB else (K, N)
    lda, ldb, ldc = ac + pad, bc + pad, N + pad
    sA, sB, sC = ar * lda + (4 if aligned else 5), br * ldb + (8 if aligned else 7), M * ldc + (4 if aligned else 2)
    offs = (0, 0, 0) if aligned else (1, 2, 3)
    return BatchedGemm(f"small_{opA}{opB}{'a' if aligned else 'u'}", batch, M, N, K, 1.25, opA, opB,
                       "a", offs[0], lda, sA, "b", offs[1], ldb, sB,
                       1 + (batch * sC + 16) // (N + pad), N + pad, offs[2], ldc, sC)


def small_buffers(prob, seed, dist="normal"):
    """Buffers that hold every batch's operands (A and B) and C's initial values."""
    rng = np.random.default_rng(seed)
    ar = (prob.K if prob.opA else prob.M)
    br = (prob.N if prob.opB else prob.K)
    a = draw(rng, (prob.a_off + prob.batch * prob.sA + ar * prob.lda,), dist)
    b = draw(rng, (prob.b_off + prob.batch * prob.sB + br * prob.ldb,), dist)
    c = draw(rng, (prob.c_rows * prob.c_cols,), "uniform")
    return {"a": a, "b": b}, c


@pytest.mark.parametrize("aligned", [False, True])
def test_every_config_every_operand_form(aligned):
    import tiled_fp32_gemm_02_amd as sg
    names = sg.configs()
    for opA, opB in OPS:
        prob = small_problem(opA, opB, aligned=aligned)
        bufs, c = small_buffers(prob, 31 + 2 * opA + opB)
        for cid, name in enumerate(names):
            if name.startswith(("sk_", "sk16_")):
                continue
            say(f"batched op {opA}{opB} aligned {aligned} config {cid} {name}")
            st, out, c0, unchanged = run_batched(prob, bufs, config=cid, c_init=c)
            assert st == 0 and all(unchanged.values()), (name, st, unchanged)
            check_batches(prob, bufs, out, c0, beta=0.5)


def test_small_integers_exact_every_form():
    """Integer entries in [-8, 8]: every partial sum is exact in fp32, so each batch must
    equal the integer product bitwise, whatever the kernel's summation order."""
    import tiled_fp32_gemm_02_amd as sg
    for opA, opB in OPS:
        prob = small_problem(opA, opB, batch=4, M=67, N=130, K=129, pad=1, aligned=opA == opB)
        bufs, _ = small_buffers(prob, 41 + opA + 2 * opB, "smallint")
        for cid in (-1, sg.configs().index("mfma_64x64x32_w2x2k2d"), 0):
            say(f"batched exact op {opA}{opB} config {cid}")
            st, out, c0, unchanged = run_batched(prob, bufs, config=cid)
            assert st == 0 and all(unchanged.values())
            for b in range(prob.batch):
                a = bufs["a"][prob.a_off + b * prob.sA:]
                bb = bufs["b"][prob.b_off + b * prob.sB:]
                ar, ac = (prob.K, prob.M) if opA else (prob.M, prob.K)
                br, bc = (prob.N, prob.K) if opB else (prob.K, prob.N)
                A = np.stack([a[r * prob.lda: r * prob.lda + ac] for r in range(ar)]).astype(np.int64)
                B = np.stack([bb[r * prob.ldb: r * prob.ldb + bc] for r in range(br)]).astype(np.int64)
                exact = ((A.T if opA else A) @ (B.T if opB else B)) * 1.25
                idx = prob.c_off + b * prob.sC + np.arange(prob.M)[:, None] * prob.ldc + np.arange(prob.N)[None, :]
                assert np.array_equal(out[idx], exact.astype(np.float32)), (opA, opB, cid, b)


def test_batched_bias_gelu():
    """A batched linear layer: the bias (shared by the batches) and tanh GELU fused."""
    prob = small_problem(0, 1, batch=5, M=96, N=200, K=64, pad=0)
    bufs, _ = small_buffers(prob, 53)
    bias = draw(np.random.default_rng(54), (prob.N,), "normal")
    say("batched bias + gelu")
    st, out, c0, unchanged = run_batched(prob, bufs, bias=bias, act=oracle.ACT_GELU_TANH)
    assert st == 0 and all(unchanged.values())
    check_batches(prob, bufs, out, c0, bias=bias, act=oracle.ACT_GELU_TANH)


def test_tensor_form_attention_views():
    """gemm_batched() on the tensor views attention uses: per-head slices of QKV, K
    transposed, and the output heads side by side, all without copies."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    T, H, D = 256, 4, 64
    bufs = gpt2_attention_set(seed=61, T=T, heads=H, hd=D)
    qkv = torch.from_numpy(bufs["qkv"]).cuda()
    p = torch.from_numpy(bufs["p"]).cuda()
    q = qkv[:, :H * D].view(T, H, D).transpose(0, 1)
    k = qkv[:, H * D:2 * H * D].view(T, H, D).transpose(0, 1)
    v = qkv[:, 2 * H * D:].view(T, H, D).transpose(0, 1)
    out = torch.empty(T, H * D, device="cuda")
    say("tensor-form attention views")
    s = sg.gemm_batched(q, k.transpose(1, 2), alpha=1.0 / 8)
    sg.gemm_batched(p, v, out.view(T, H, D).transpose(0, 1))
    torch.cuda.synchronize()
    s_np, out_np = s.cpu().numpy(), out.cpu().numpy()
    w = 3 * H * D
    flat = bufs["qkv"].reshape(-1)
    for h in range(H):
        ref, bound = oracle.gemm(0, 1, T, T, D, 1.0 / 8, flat[h * D:], w, flat[H * D + h * D:], w, 0.0, None, T)
        assert oracle.within_bound(s_np[h], ref, bound)[0], h
        ref, bound = oracle.gemm(0, 0, T, D, T, 1.0, bufs["p"][h], T, flat[2 * H * D + h * D:], w, 0.0, None, D)
        assert oracle.within_bound(out_np[:, h * D:(h + 1) * D], ref, bound)[0], h
