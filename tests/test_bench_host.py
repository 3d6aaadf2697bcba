"""Host-side pieces of bench.py and the sweep (CPU only): the one-GPU guard, the sysfs
clock reader, the oracle's bounded CPU sample and the sweep's argument handling."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import Gemm, make  # noqa: E402

def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

def test_read_sclk_is_an_int_or_none():
    v = bench.read_sclk()
    assert v is None or (isinstance(v, int) and v > 0)

def _host_linear(w):
    """A LinearProblem's host half (inputs, oracle leg) without device copies."""
    p = bench.LinearProblem.__new__(bench.LinearProblem)
    p.w, p.name, p.M, p.N, p.K, p.batch = w, w.name, w.M, w.N, w.K, 1
    p.A, p.B, p.C = make(w)
    p.bias, p.act = None, 0
    return p


def _host_batched(prob, bufs):
    p = bench.BatchedProblem.__new__(bench.BatchedProblem)
    p.p, p.name, p.M, p.N, p.K, p.batch, p.bufs = prob, prob.name, prob.M, prob.N, prob.K, prob.batch, bufs
    return p


def test_cpu_baseline_samples_every_product():
    from workloads import attention_products, gpt2_attention_set
    probs = [_host_linear(Gemm(name, M, N, K, alpha=1.5, beta=0.5, seed=7))
             for name, (M, N, K) in {"p1": (64, 48, 40), "p2": (32, 80, 24)}.items()]
    out = bench.cpu_baseline(probs, 0.05)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["cores"] >= 1
    assert "64x48x40" in out["sample"] and "32x80x24" in out["sample"]
    bufs = gpt2_attention_set(seed=3, T=64, heads=3, hd=16)
    out = bench.cpu_baseline([_host_batched(p, bufs) for p in attention_products(T=64, heads=3, hd=16)], 0.05)
    assert out["value"] > 0 and "each of the 3 64x64x16 products" in out["sample"]

def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; } // one\n/* block */\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setattr(bench, "MFMA_KERNEL_SOURCES", ("k.hip",))
    h1 = bench.kernel_source_hash()
    src.write_text("int f() {   return 1; }   // a different comment\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_sweep_parses_shapes_and_needs_a_gpu(monkeypatch):
    from tiled_fp32_gemm_02_amd import sweep
    assert sweep.parse_shapes("4096,4096,4096;1,2,3") == [(4096, 4096, 4096), (1, 2, 3)]
    import torch
    monkeypatch.setattr(torch.cuda, "is_available", lambda: False)
    with pytest.raises(SystemExit):
        sweep.main(["--shapes", "64,64,64", "--configs", "0"])


def test_tile_traffic_model():
    """The tiles' operand-panel bytes: 4 M N K (1/BM + 1/BN), from the configuration's name."""
    import bench
    assert bench.tile_dims("mfma_256x256x32_w2x4d") == (256, 256)
    assert bench.tile_dims("mfma_32x128x64_w1x4k2d") == (32, 128)
    assert bench.tile_dims("sk_64x128x32_w2x2k2p2") == (64, 128)
    assert bench.tile_dims("valu_128x128x8_t8x8") == (128, 128)
    assert bench.tile_dims("tile16") == (16, 16)
    # 4096^3 on 256 x 256 tiles: 2 * 4096^3 * 4 / 256 bytes
    assert bench.lds_fill_bytes(4096, 4096, 4096, "mfma_256x256x32_w2x4d") == 2 * 4 * 4096 ** 3 / 256
    # 16 x 16 tiles read MNK/8 floats (AutoMine++ #4, section "current algorithm")
    assert bench.lds_fill_bytes(64, 64, 64, "tile16") == 4 * 64 ** 3 / 8
    import tiled_fp32_gemm_02_amd as sg
    for name in sg.configs():
        bench.tile_dims(name)


def test_register_tile_and_clock_peak():
    """The LDS -> register model uses the wave tile (matrix cores) or the thread's micro-tile;
    the clock-adjusted peak is CUs x 256 flop/clk x sclk."""
    assert bench.register_tile("mfma_256x256x32_w2x4d") == (128, 64)
    assert bench.register_tile("mfma_32x128x64_w1x4k2d") == (32, 32)
    assert bench.register_tile("sk_64x128x32_w2x2k2p2") == (32, 64)
    assert bench.register_tile("valu_128x128x8_t8x8") == (8, 8)
    assert bench.register_tile("tile16") == (1, 1)
    # one output per thread: two LDS reads per multiply-add
    assert bench.lds_read_bytes(64, 64, 64, "tile16") == 4 * 2 * 64 ** 3
    assert bench.lds_read_bytes(4096, 4096, 4096, "mfma_256x256x32_w2x4d") == 4 * 4096 ** 3 * (1 / 128 + 1 / 64)
    # 256 CUs at 2.4 GHz: the published 157.3 TFLOP/s
    assert abs(bench.peak_at_clock(256, 2400) - 157.2864) < 1e-9
    assert bench.peak_at_clock(256, None) is None
    import tiled_fp32_gemm_02_amd as sg
    for name in sg.configs():
        tm, tn = bench.register_tile(name)
        assert tm >= 1 and tn >= 1
