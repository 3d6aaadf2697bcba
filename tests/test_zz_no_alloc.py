"""GPU checks of the allocation-free entry point, sgemm_general_noalloc, through the C ABI.

Its output must equal that of sgemm_general_ws (the entry point it is a variant of) on the
same inputs, and match the oracle within the error bound, on two calls in a row on one
stream, the second with a smaller input: the scratch array keeps the first call's
contents, and the second must not be affected by them. The shapes are ones the cost model
sends to stream-K (which uses the scratch); a forced data-parallel configuration and the
unaligned path (stream-K configurations then run their tile kernel) are covered too.
"""

import numpy as np
import pytest

import oracle
from gpu_util import say
from workloads import draw

pytestmark = pytest.mark.gpu

COUNTER_WORDS = 16384


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    sgbuild.ensure_built()
    import tiled_fp32_gemm_02_amd as sg
    sg.load()


def _pair(config, M, N, K, seed, ws, offset=0):
    """One product through both entry points on the current stream; returns the two C
    windows, the oracle's (ref, bound) and the configuration names the library picks."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    rng = np.random.default_rng(seed)
    a, b, c = draw(rng, (M, K), "normal"), draw(rng, (K, N), "normal002"), draw(rng, (M, N), "uniform")
    bias = draw(rng, (N,), "normal")
    dA = torch.from_numpy(np.concatenate([np.zeros(offset, np.float32), a.reshape(-1)])).cuda()
    dB = torch.from_numpy(b).cuda()
    dbias = torch.from_numpy(bias).cuda()
    outs = []
    for which in ("ws", "noalloc"):
        dC = torch.from_numpy(c).cuda()
        pa = dA.data_ptr() + 4 * offset
        s = torch.cuda.current_stream()
        say(f"{which} config {config} {M}x{N}x{K} offset {offset}")
        if which == "ws":
            st = sg.sgemm_general_ws(config, 0, 0, M, N, K, 1.5, pa, K, dB, N, 0.5, dC, N, dbias, 0, ws,
                                     ws.numel(), s)
        else:
            st = sg.sgemm_general_noalloc(config, 0, 0, M, N, K, 1.5, pa, K, dB, N, 0.5, dC, N, dbias, 0, s)
        assert st == 0, (which, st, sg.sgemm_status_string(st))
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
    ref, bound = oracle.gemm(0, 0, M, N, K, 1.5, a, K, b, N, 0.5, c, N, bias)
    pick = sg.sgemm_config_name(config) if config >= 0 else sg.sgemm_config_name(
        sg.sgemm_select_config_general(0, 0, M, N, K, 1.5, pa, K, 0, dB, N, 0, dC, N, 0, 1,
                                       sg.SGEMM_NOALLOC_SCRATCH_BYTES))
    return outs, ref, bound, pick


def _check(outs, ref, bound):
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "noalloc differs from the ws call"
    for out in outs:
        ok, worst, idx = oracle.within_bound(out, ref, bound)
        assert ok, (worst, idx)


def test_noalloc_matches_the_workspace_entry_point():
    """Two calls in a row, the second smaller, automatic choice: both stream-K."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    ws = torch.zeros(sg.sgemm_workspace_size(-1), dtype=torch.uint8, device="cuda")
    assert ws.numel() <= sg.SGEMM_NOALLOC_SCRATCH_BYTES
    picks = []
    for (M, N, K), seed in (((2560, 2560, 2560), 1), ((512, 512, 8192), 2)):
        outs, ref, bound, pick = _pair(-1, M, N, K, seed, ws)
        _check(outs, ref, bound)
        picks.append(pick)
    assert all(p.startswith(("sk_", "sk16_")) for p in picks), picks


def test_noalloc_forced_configurations():
    """Every stream-K configuration, a data-parallel one and the unaligned path, each on
    two calls in a row with the second smaller."""
    import torch
    import tiled_fp32_gemm_02_amd as sg
    ws = torch.zeros(sg.sgemm_workspace_size(-1), dtype=torch.uint8, device="cuda")
    names = sg.configs()
    ids = [i for i, n in enumerate(names) if n.startswith(("sk_", "sk16_"))] + [names.index("mfma_64x64x32_w2x2k2d")]
    for cid in ids:
        for (M, N, K), seed, offset in (((1100, 1300, 1028), 3, 0), ((300, 260, 132), 4, 0),
                                        ((257, 255, 131), 5, 1)):
            outs, ref, bound, _ = _pair(cid, M, N, K, seed + cid, ws, offset)
            _check(outs, ref, bound)
