"""The C-ABI library on the CPU: it loads, exports every function include/sgemm.h
declares, and its host logic (argument validation, quick returns, configuration
choice, launch shapes) behaves as documented. No call here reaches a kernel
launch: every case is rejected or returns before touching the GPU.
"""

import os
import re

import pytest

import tiled_fp32_gemm_02_amd as sg
from tiled_fp32_gemm_02_amd import build as sgbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")
BAD = 0xDEAD0  # a pointer value that must never be dereferenced in these tests


@pytest.fixture(scope="module", autouse=True)
def _built():
    sgbuild.ensure_built()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_exports_every_declared_function():
    import ctypes
    lib = ctypes.CDLL(sg.lib_path())
    names = declared_functions()
    assert set(names) == set(sg.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), f"libsgemm.so does not export {name}"


def test_version_and_configs():
    assert "gfx950" in sg.sgemm_version()
    names = sg.configs()
    assert len(names) == sg.sgemm_config_count() >= 2
    assert names[0] == "tile16"
    # matrix-core configurations first, then the stream-K ones, then the vector-ALU micro-tile
    kinds = [n.split("_")[0] for n in names[1:]]
    assert set(kinds) == {"mfma", "mfma16", "sk", "sk16", "valu"} and kinds == sorted(kinds)
    assert sg.sgemm_config_name(-1) is None and sg.sgemm_config_name(len(names)) is None


@pytest.mark.parametrize("args,code", [
    # (M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    ((-1, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -1),
    ((4, -1, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -2),
    ((4, 4, -1, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -3),
    ((4, 4, 4, 1.0, None, 4, BAD, 4, 0.0, BAD, 4), -5),
    ((4, 4, 8, 1.0, BAD, 7, BAD, 4, 0.0, BAD, 4), -6),
    ((4, 4, 0, 1.0, BAD, 0, BAD, 4, 0.0, BAD, 4), -6),   # lda >= max(1, K)
    ((4, 4, 4, 1.0, BAD, 4, None, 4, 0.0, BAD, 4), -7),
    ((4, 5, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 5), -8),
    ((4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, None, 4), -10),
    ((4, 5, 4, 1.0, BAD, 4, BAD, 5, 0.0, BAD, 4), -11),
    ((4, 0, 4, 1.0, BAD, 4, BAD, 0, 0.0, BAD, 1), -8),   # ldb >= 1 even when N == 0
])
def test_invalid_arguments(args, code):
    assert sg.sgemm(*args) == code
    assert sg.sgemm_ex(-1, *args) == code
    assert sg.sgemm_status_string(code) == f"invalid argument {-code}"


def test_first_invalid_argument_wins():
    assert sg.sgemm(-1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0) == -1
    assert sg.sgemm(3, 3, -1, 1.0, None, 0, None, 0, 0.0, None, 0) == -3


def test_null_pointers_allowed_when_unread():
    # empty result: nothing is touched
    assert sg.sgemm(0, 7, 5, 1.0, None, 5, None, 7, 0.5, None, 7) == 0
    assert sg.sgemm(7, 0, 5, 1.0, None, 5, None, 1, 0.5, None, 1) == 0
    # A and B unread when alpha == 0 or K == 0, but C is still required
    assert sg.sgemm(4, 4, 0, 1.0, None, 1, None, 4, 0.0, None, 4) == -10
    assert sg.sgemm(4, 4, 3, 0.0, None, 3, None, 4, 0.0, None, 4) == -10


def test_bad_config_id():
    args = (4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4)
    assert sg.sgemm_ex(-2, *args) == sg.SGEMM_ERROR_BAD_CONFIG
    assert sg.sgemm_ex(sg.sgemm_config_count(), *args) == sg.SGEMM_ERROR_BAD_CONFIG
    assert "configuration" in sg.sgemm_status_string(sg.SGEMM_ERROR_BAD_CONFIG)


@pytest.mark.parametrize("args,code", [
    # (M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch)
    ((-1, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -1),
    ((4, 4, 4, 1.0, None, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -5),
    ((4, 4, 8, 1.0, BAD, 7, 32, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -6),
    ((4, 4, 4, 1.0, BAD, 4, -1, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -7),
    ((4, 4, 4, 1.0, BAD, 4, 16, None, 4, 16, 0.0, BAD, 4, 16, 2), -8),
    ((4, 5, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 5, 20, 2), -9),
    ((4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, -4, 0.0, BAD, 4, 16, 2), -10),
    ((4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, None, 4, 16, 2), -12),
    ((4, 5, 4, 1.0, BAD, 4, 16, BAD, 5, 20, 0.0, BAD, 4, 20, 2), -13),
    ((4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 15, 2), -14),  # C windows overlap
    ((4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, -1), -15),
    ((4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 65536), -15),
])
def test_batched_invalid_arguments(args, code):
    assert sg.sgemm_strided_batched(*args) == code


@pytest.mark.parametrize("args,code", [
    # (opA, opB, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch)
    ((2, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -1),
    ((0, 3, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -2),
    ((0, 0, -1, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -3),
    ((0, 0, 4, 4, 4, 1.0, None, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -7),
    ((1, 0, 6, 4, 8, 1.0, BAD, 5, 48, BAD, 4, 32, 0.0, BAD, 4, 24, 2), -8),      # transposed A: lda >= M
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, -4, BAD, 4, 16, 0.0, BAD, 4, 16, 2), -9),
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, None, 4, 16, 0.0, BAD, 4, 16, 2), -10),
    ((0, 1, 4, 6, 8, 1.0, BAD, 8, 32, BAD, 7, 48, 0.0, BAD, 6, 24, 2), -11),     # transposed B: ldb >= K
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, -1, 0.0, BAD, 4, 16, 2), -12),
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, None, 4, 16, 2), -14),
    ((0, 0, 4, 5, 4, 1.0, BAD, 4, 16, BAD, 5, 20, 0.0, BAD, 4, 20, 2), -15),
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 15, 2), -16),     # C windows overlap
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, -16, 2), -16),
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 12, 4, 4), -16),     # side by side: 4 x 4 > 12
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 12, 3, 3), -16),     # side by side, overlapping
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, -1), -17),
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 65536), -17),
])
def test_batched_op_invalid_arguments(args, code):
    assert sg.sgemm_strided_batched_op(*args) == code
    # the general form: same positions up to C's stride; bias and act come before batch
    gen = args[:16] + (None, sg.SGEMM_ACT_NONE, args[16])
    expect = code if code > -17 else -19
    assert sg.sgemm_strided_batched_general(-1, *gen) == expect
    assert sg.sgemm_status_string(code) == f"invalid argument {-code}"


def test_batched_strides_bounded():
    """(batch - 1) * stride past 2^60 floats is rejected at that stride's position."""
    big = (1 << 60) // 2 + 1
    assert sg.sgemm_strided_batched(4, 4, 4, 1.0, BAD, 4, big, BAD, 4, 16, 0.0, BAD, 4, 16, 3, None) == -7
    assert sg.sgemm_strided_batched(4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, big, 0.0, BAD, 4, 16, 3, None) == -10
    assert sg.sgemm_strided_batched(4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, big, 3, None) == -14
    # one batch: the stride is never applied
    assert sg.sgemm_strided_batched(0, 4, 4, 1.0, BAD, 4, 1 << 62, BAD, 4, 16, 0.0, BAD, 4, 16, 1, None) == 0


def test_batched_general_checks():
    ok = (0, 0, 4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16)
    assert sg.sgemm_strided_batched_general(-1, *ok, None, 2, 2) == -18          # act
    assert sg.sgemm_strided_batched_general(-2, *ok, None, 0, 2) == sg.SGEMM_ERROR_BAD_CONFIG
    sk = [i for i, n in enumerate(sg.configs()) if n.startswith(("sk_", "sk16_"))]
    assert sg.sgemm_strided_batched_general(sk[0], *ok, None, 0, 2) == sg.SGEMM_ERROR_WORKSPACE
    # quick returns: nothing launched, unread pointers may be anything
    assert sg.sgemm_strided_batched_general(-1, *ok, None, 0, 0) == 0
    assert sg.sgemm_strided_batched_op(0, 0, 0, 4, 4, 1.0, None, 4, 0, None, 4, 0, 0.0, None, 4, 0, 9) == 0
    assert sg.sgemm_status_string(-20) == "invalid argument 20"


def test_batched_side_by_side_windows_accepted():
    """Heads written side by side into the rows of one matrix (attention's output): each
    window N wide, all within ldc. Accepted by the plain batched form too; the call here
    stops before any launch because batch == 0 after the checks would launch nothing, so
    the acceptance is seen through the quick return of M == 0."""
    # 12 heads of 64 columns in a 768-wide row: accepted (the M == 0 quick return follows)
    assert sg.sgemm_strided_batched(0, 64, 1024, 1.0, None, 1024, 0, None, 64, 0, 0.0, None, 768, 64, 12) == 0
    assert sg.sgemm_strided_batched_op(0, 0, 0, 64, 1024, 1.0, None, 1024, 0, None, 64, 0, 0.0, None, 768, 64,
                                       12) == 0
    # one column too many for the row: rejected before the quick return is reached
    args = (5, 64, 16, 1.0, BAD, 16, 0, BAD, 64, 0, 0.0, BAD, 767, 64, 12)
    assert sg.sgemm_strided_batched(*args) == -14
    assert sg.sgemm_strided_batched_op(0, 0, *args) == -16


def test_batched_quick_returns():
    assert sg.sgemm_strided_batched(4, 4, 4, 1.0, BAD, 4, 16, BAD, 4, 16, 0.0, BAD, 4, 16, 0) == 0
    assert sg.sgemm_strided_batched(0, 4, 4, 1.0, None, 4, 0, None, 4, 0, 0.0, None, 4, 0, 9) == 0


def test_launch_shape_tile16_matches_gpt2_post():
    # The GPT-2 post covers a 64 x 256 matrix with a 4 x 16 grid of 16 x 16-thread
    # blocks ("GPU Target", section "From loops to kernels"); its matmul kernel puts n
    # on grid x and m on grid y ("Tiled matrix multiplication"), both ceil-divided.
    assert sg.sgemm_launch_shape(0, 64, 256, 16) == (0, (16, 4, 1), (16, 16, 1))
    assert sg.sgemm_launch_shape(0, 65, 257, 3) == (0, (17, 5, 1), (16, 16, 1))
    assert sg.sgemm_launch_shape(0, 1, 1, 1) == (0, (1, 1, 1), (16, 16, 1))


def test_launch_shape_valu():
    cid = sg.configs().index("valu_128x128x8_t8x8")
    for M, N in [(4096, 4096), (1000, 1537), (1, 1), (129, 127)]:
        assert sg.sgemm_launch_shape(cid, M, N, 64) == (0, (-(-M // 128) * -(-N // 128), 1, 1), (256, 1, 1))


def test_launch_shape_mfma():
    for cid, name in enumerate(sg.configs()):
        if not name.startswith(("mfma_", "mfma16_")):
            continue
        m = re.fullmatch(r"mfma(?:16)?_(\d+)x(\d+)x(\d+)_w(\d+)x(\d+)(?:k(\d+))?(?:p(\d+))?(d)?", name)
        assert m, name
        bm, bn, _, wm, wn = (int(x) for x in m.groups()[:5])
        wk = int(m.group(6) or 1)
        for M, N in [(4096, 4096), (1000, 1537), (1, 1), (bm + 1, bn - 1)]:
            st, grid, block = sg.sgemm_launch_shape(cid, M, N, 64)
            assert st == 0
            tiles = -(-M // bm) * -(-N // bn)
            whole = -(-M // bm) * (N // bn)
            if 1 <= N % bn <= 8 and whole >= 256:       # fringe columns: whole tiles + two rows each
                tiles = whole + -(-M // 2)
            assert grid == (tiles, 1, 1)
            assert block == (wm * wn * wk * 64, 1, 1)
        assert sg.sgemm_launch_shape(cid, -1, 4, 4)[0] == -1
    st, _, _ = sg.sgemm_launch_shape(1, 2**31 - 1, 2**31 - 1, 1)
    assert st == sg.SGEMM_ERROR_TOO_LARGE
    assert sg.sgemm_launch_shape(99, 4, 4, 4)[0] == sg.SGEMM_ERROR_BAD_CONFIG


def test_launch_shape_near_int_max():
    """Sizes within one tile of 2^31: the ceiling divisions must not overflow. Each
    launch is either described exactly or rejected as too large."""
    big = 2**31 - 1
    # 16x16 kernel: a 2-D grid of 16x16 blocks over N x M
    assert sg.sgemm_launch_shape(0, big, 1, big) == (0, (1, 2**27, 1), (16, 16, 1))
    assert sg.sgemm_launch_shape(0, 1, big, 1) == (0, (2**27, 1, 1), (16, 16, 1))
    valu = sg.configs().index("valu_128x128x8_t8x8")
    # ceil(big / 128) x 256 threads is 2^32: one more than a launch holds
    assert sg.sgemm_launch_shape(valu, big, 1, 8)[0] == sg.SGEMM_ERROR_TOO_LARGE
    m = big - 128
    assert sg.sgemm_launch_shape(valu, m, 1, 8) == (0, (-(-m // 128), 1, 1), (256, 1, 1))
    for cid, name in enumerate(sg.configs()):
        if name.startswith(("mfma_", "mfma16_")):
            st, grid, block = sg.sgemm_launch_shape(cid, big, 1, big)
            bm = int(name.split("_")[1].split("x")[0])
            fits = -(-big // bm) * block[0] <= 2**32 - 1 if st == 0 else False
            assert st == (0 if fits else sg.SGEMM_ERROR_TOO_LARGE), (name, st)
            if st == 0:
                assert grid == (-(-big // bm), 1, 1)
        elif name.startswith(("sk_", "sk16_")):
            # K-tile steps x (compute units + 1) pass 2^31
            assert sg.sgemm_launch_shape(cid, 64, 64, big)[0] == sg.SGEMM_ERROR_TOO_LARGE, name


def test_select_config_near_int_max():
    names = sg.configs()
    big = 2**31 - 1
    for M, N, K in [(1, 1, big), (big, 1, 1), (1, big, 1), (big - 128, 1, 4)]:
        cid = sg.sgemm_select_config(M, N, K, 1.0, BAD, max(K, 1), BAD, N, BAD, N)
        assert 0 <= cid < len(names), (M, N, K, cid)


def test_select_config():
    names = sg.configs()
    sel = lambda M, N, K=64, alpha=1.0: sg.sgemm_select_config(M, N, K, alpha, BAD, K, BAD, N, BAD, N)
    assert sel(0, 5) == -1 and sel(5, 0) == -1 and sel(5, 5, K=0) == -1 and sel(5, 5, alpha=0.0) == -1
    assert names[sel(4096, 4096, 4096)] == "mfma_256x256x32_w2x4d"    # 256 tiles: one per CU
    # rows only 4-byte aligned: the unaligned table, whose large tiles have 4-byte-copy forms
    assert names[sg.sgemm_select_config(4096, 4096, 4096, 1.0, BAD + 4, 4096, BAD, 4096, BAD, 4096)] == \
        "mfma_256x256x16_w2x4p2d"
    assert names[sel(4095, 4095, 4095)] == "mfma_256x256x16_w2x4p2d"
    # each choice still gives at least 256 workgroups when the problem allows it
    for M, N in [(1024, 1024), (1024, 2304), (1024, 3072), (1024, 768), (1000, 1537), (256, 256)]:
        name = names[sel(M, N)]
        bm, bn, _ = (int(x) for x in name.split("_")[1].split("x"))
        tiles = -(-M // bm) * -(-N // bn)
        assert tiles >= 256 or bm <= 64, (M, N, name, tiles)
    # the modelled winners without a workspace: 16x16-block tiles for the GPT-2 QKV layer and
    # 1536^3 (32 x 96: three tiles per CU), the MLP-up layer, 1024^3, 256^3 (whole K in one
    # 256-deep K-tile) and the 32-wide and 32-row products; the 32x32-block tile for MLP-down
    assert names[sel(1024, 2304, 768)] == "mfma16_32x96x64_w2x2k2d"
    assert names[sel(1536, 1536, 1536)] == "mfma16_32x96x64_w2x2k2d"
    assert names[sel(1024, 3072, 768)] == "mfma16_64x64x32_w4x1k1d"
    assert names[sel(1024, 768, 3072)] == "mfma_32x32x64_w1x1k4d"
    assert names[sel(1024, 1024, 1024)] == "mfma16_64x64x64_w4x1k2d"
    assert names[sel(256, 256, 256)] == "mfma16_16x16x256_w1x1k4d"
    assert names[sel(8192, 32, 8192)] == "mfma16_32x32x128_w2x2k2d"
    assert names[sel(32, 8192, 8192)] == "mfma16_32x32x128_w2x2k2d"
    # unaligned: the ragged product on the 32 x 64 16x16-block tile, 32 x 24 whole tiles (three
    # per CU) and one fringe column
    assert names[sg.sgemm_select_config(1000, 1537, 777, 1.0, BAD, 777, BAD, 1537, BAD, 1537)] == \
        "mfma16_32x64x64_w2x1k2d"


def test_config_describe_every_id():
    """Every configuration has one description line whose fields agree with its name,
    its launch shape and the limits of the hardware; ids out of range give NULL."""
    names = sg.configs()
    kinds = {"tile16": "tile16", "mfma": "mfma", "mfma16": "mfma", "sk": "streamk", "sk16": "streamk", "valu": "valu"}
    for cid, name in enumerate(names):
        d = sg.describe(cid)
        assert set(d) == {"name", "kind", "tile", "waves", "kgroups", "threads", "ahead", "loader", "lds_bytes",
                          "band", "unaligned", "unaligned_bk", "compute"}, d
        assert d["name"] == name and d["kind"] == kinds[name.split("_")[0]]
        bm, bn, bk = (int(x) for x in d["tile"].split("x"))
        wm, wn = (int(x) for x in d["waves"].split("x"))
        wk, threads, lds = int(d["kgroups"]), int(d["threads"]), int(d["lds_bytes"])
        assert 0 < lds <= 160 * 1024 and int(d["band"]) >= 1 and int(d["unaligned_bk"]) >= 1
        if d["kind"] in ("mfma", "streamk"):
            m = re.fullmatch(r"(mfma|mfma16|sk|sk16)_(\d+)x(\d+)x(\d+)_w(\d+)x(\d+)(?:k(\d+))?(?:p(\d+))?(d)?", name)
            assert m, name
            assert (bm, bn, bk, wm, wn) == tuple(int(x) for x in m.groups()[1:6])
            assert wk == int(m.group(7) or 1) and int(d["ahead"]) == int(m.group(8) or 1)
            assert threads == wm * wn * wk * 64
            assert d["loader"] == ("direct-16B" if m.group(9) else "staged-16B")
            assert d["compute"] == ("v_mfma_f32_16x16x4_f32" if m.group(1) in ("mfma16", "sk16") else "v_mfma_f32_32x32x2_f32")
            # the stages hold A and B tiles: at least BK * (BM + BN) floats per stage
            assert lds >= 4 * bk * (bm + bn)
        if d["kind"] in ("mfma", "streamk"):
            # direct-copy configurations keep their copies and K-tile on 4-byte aligned rows
            direct = d["loader"] == "direct-16B"
            assert d["unaligned"] == ("direct-16B-unaligned" if direct else
                                      "data-parallel-staged-4B" if d["kind"] == "streamk" else "staged-4B")
            assert int(d["unaligned_bk"]) == bk
        if d["kind"] != "streamk":
            st, grid, block = sg.sgemm_launch_shape(cid, 1000, 1537, 777)
            assert st == 0 and block[0] * block[1] * block[2] == threads
    for bad in (-1, -2, len(names), len(names) + 7, 2**31 - 1):
        assert sg.sgemm_config_describe(bad) is None
        with pytest.raises(ValueError):
            sg.describe(bad)
    # the direct-copy large tile: 2 stages of (256 + 256) x 32 floats
    d = sg.describe(names.index("mfma_256x256x32_w2x4d"))
    assert d["lds_bytes"] == str(2 * 32 * 512 * 4) and d["unaligned"] == "direct-16B-unaligned"


def test_select_config_repeats_and_interleaves():
    """The host keeps a small memo of recent choices per thread: the pick for a shape is the
    same however queries for other shapes (more than the memo holds) and alignments are
    interleaved with it."""
    names = sg.configs()
    shapes = [(256, 256, 256), (1024, 2304, 768), (4096, 4096, 4096), (1000, 1537, 777), (1024, 768, 3072),
              (8192, 32, 8192), (32, 8192, 8192), (1536, 1536, 1536), (3000, 3000, 3000), (16, 16384, 16384),
              (1024, 1024, 64), (512, 512, 8192)]
    def pick(M, N, K, lda, ws):
        return sg.sgemm_select_config_ws(M, N, K, 1.0, BAD, lda, BAD, N, BAD, N, ws)
    first = {(s, a, w): pick(*s, s[2] + a, w) for s in shapes for a in (0, 1) for w in (0, 1 << 26)}
    rng = __import__("random").Random(3)
    keys = list(first) * 3
    rng.shuffle(keys)
    for (s, a, w) in keys:
        assert pick(*s, s[2] + a, w) == first[(s, a, w)], (s, a, w)
    assert names[first[((4096, 4096, 4096), 0, 0)]] == "mfma_256x256x32_w2x4d"


def test_batched_products_take_the_batched_list():
    """Strided-batched products choose among the tiles fitted on batched shapes: the 64 x 128
    16x16-block tile for attention's scores (12 x 1024^2 x 64, K transposed) and the short-K
    forms, the 16 x 64 one for its values (12 x 1024 x 64 x 1024); never the 256-wide tiles,
    which a 12 x 1024^2 x 16 product once took from the single-product list. Unaligned
    operands (odd row lengths) use the same list, not the unaligned single-product one, whose
    128 x 128 tile ran 5-47% behind these on attention-like shapes."""
    names = sg.configs()
    def sel(b, M, N, K, opB):
        return names[sg.sgemm_select_config_general(0, opB, M, N, K, 1.0, BAD, K, M * K, BAD, K if opB else N, K * N,
                                                    BAD, N, M * N, b)]
    assert sel(12, 1024, 1024, 64, 1) == "mfma16_64x128x32_w4x2k1d"
    assert sel(12, 1024, 64, 1024, 0) == "mfma16_16x64x64_w1x1k4d"
    for K in (16, 32, 128, 256):
        assert sel(12, 1024, 1024, K, 1) == "mfma16_64x128x32_w4x2k1d"
    assert sel(1, 1024, 1024, 1024, 0) == "mfma16_64x64x64_w4x1k2d"     # one product: the single list
    # rows only 4-byte aligned (odd K or N) take the same list, run with unaligned direct copies
    assert sel(12, 1024, 1024, 63, 1) == "mfma16_64x128x32_w4x2k1d"
    assert sel(12, 1023, 1023, 127, 1) == "mfma16_64x128x32_w4x2k1d"
    assert sel(12, 1023, 63, 1023, 0) == "mfma16_16x64x64_w1x1k4d"
    assert sel(12, 1024, 65, 2047, 0) == "mfma16_32x32x64_w2x2k1d"


def test_select_config_general_agrees_with_the_plain_query():
    """batch == 1 with plain operands: the same pick as sgemm_select_config; the batch
    multiplies the tile count the cost model spreads over the compute units."""
    names = sg.configs()
    for M, N, K in [(4096, 4096, 4096), (1024, 2304, 768), (1000, 1537, 777), (256, 256, 256), (1, 1, 1)]:
        for a in (BAD, BAD + 4):
            plain = sg.sgemm_select_config(M, N, K, 1.0, a, K, BAD, N, BAD, N)
            assert sg.sgemm_select_config_general(0, 0, M, N, K, 1.0, a, K, 0, BAD, N, 0, BAD, N, 0, 1, 0) == plain
    assert sg.sgemm_select_config_general(0, 0, 64, 64, 64, 0.0, BAD, 64, 0, BAD, 64, 0, BAD, 64, 0, 4, 0) == -1
    assert sg.sgemm_select_config_general(0, 0, 64, 64, 64, 1.0, BAD, 64, 0, BAD, 64, 0, BAD, 64, 0, 0, 0) == -1
    # 12 heads of 1024 x 1024 x 64: enough tiles to fill the chip with a larger tile than one head alone gets
    one = names[sg.sgemm_select_config_general(0, 1, 1024, 1024, 64, 0.125, BAD, 2304, 64, BAD, 2304, 64, BAD,
                                               1024, 1 << 20, 1, 0)]
    twelve = names[sg.sgemm_select_config_general(0, 1, 1024, 1024, 64, 0.125, BAD, 2304, 64, BAD, 2304, 64, BAD,
                                                  1024, 1 << 20, 12, 0)]
    area = lambda n: int(n.split("_")[1].split("x")[0]) * int(n.split("_")[1].split("x")[1])
    assert area(twelve) >= area(one), (one, twelve)
    # one product: a misaligned pointer takes the unaligned table
    misaligned = sg.sgemm_select_config_general(0, 0, 1024, 2304, 768, 1.0, BAD + 4, 768, 0, BAD, 2304, 0, BAD,
                                                2304, 0, 1, 0)
    aligned = sg.sgemm_select_config_general(0, 0, 1024, 2304, 768, 1.0, BAD, 768, 0, BAD, 2304, 0, BAD, 2304,
                                             0, 1, 0)
    assert misaligned != aligned, (names[misaligned], names[aligned])
    # two products, aligned or with odd strides: the batched list's tile for a few large products
    for sA in (3, 4):
        two = sg.sgemm_select_config_general(0, 0, 1024, 2304, 768, 1.0, BAD, 768, sA, BAD, 2304, 0, BAD, 2304,
                                             1 << 22, 2, 0)
        assert names[two] == "mfma16_64x96x64_w4x2k1d", (sA, names[two])


def test_status_strings():
    assert sg.sgemm_status_string(0) == "success"
    assert "too large" in sg.sgemm_status_string(sg.SGEMM_ERROR_TOO_LARGE)
    assert sg.sgemm_status_string(-99) == "unknown status"
    assert isinstance(sg.sgemm_status_string(1), str)  # a hipError_t message


def test_tensor_form_validates_before_any_launch():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 3)
    with pytest.raises(ValueError, match="Dimension error"):
        sg.gemm(torch.zeros(4), torch.zeros(4, 3))
    with pytest.raises(ValueError, match="float32"):
        sg.gemm(a.double(), torch.zeros(3, 2))
    with pytest.raises(ValueError, match="GPU"):
        sg.gemm(a, torch.zeros(3, 2))
    with pytest.raises(ValueError, match="Dimension error"):
        sg.gemm_batched(a, torch.zeros(3, 2))


@pytest.mark.parametrize("args,code", [
    # sgemm_op(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    ((2, 0, 4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -1),
    ((0, -1, 4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -2),
    ((0, 0, -1, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -3),
    ((0, 0, 4, 4, -1, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4), -5),
    ((0, 0, 4, 4, 4, 1.0, None, 4, BAD, 4, 0.0, BAD, 4), -7),
    ((1, 0, 6, 4, 8, 1.0, BAD, 5, BAD, 4, 0.0, BAD, 4), -8),     # transposed A: lda >= M
    ((0, 1, 4, 6, 8, 1.0, BAD, 8, BAD, 7, 0.0, BAD, 6), -10),    # transposed B: ldb >= K
    ((0, 0, 4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, None, 4), -12),
    ((0, 0, 4, 5, 4, 1.0, BAD, 4, BAD, 5, 0.0, BAD, 4), -13),
])
def test_op_invalid_arguments(args, code):
    assert sg.sgemm_op(*args) == code
    # the fused form numbers the same arguments the same way
    assert sg.sgemm_bias_act(*args, None, sg.SGEMM_ACT_NONE) == code


def test_bias_act_invalid_act():
    args = (0, 0, 4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4, None)
    assert sg.sgemm_bias_act(*args, 2) == -15
    assert sg.sgemm_bias_act(*args, -1) == -15
    assert sg.sgemm_general(0, *args, 7) == -15
    assert sg.sgemm_general(-2, *args, 0) == sg.SGEMM_ERROR_BAD_CONFIG


def test_op_quick_returns_touch_nothing():
    assert sg.sgemm_op(1, 1, 0, 5, 3, 1.0, None, 1, None, 3, 0.0, None, 5) == 0
    assert sg.sgemm_bias_act(1, 0, 5, 0, 3, 1.0, None, 5, None, 1, 0.0, None, 1, None, 1) == 0


def test_tensor_form_rejects_host_views():
    torch = pytest.importorskip("torch")
    x = torch.zeros(6, 4)
    with pytest.raises(ValueError, match="GPU"):
        sg.gemm(x.t(), torch.zeros(6, 3))
    with pytest.raises(ValueError, match="Dimension error"):
        sg.gemm(torch.zeros(2, 3, 4), torch.zeros(4, 3))


# --------------------------------------------------------------------------- workspace entry point

WS_ARGS = (0, 0, 4, 4, 4, 1.0, BAD, 4, BAD, 4, 0.0, BAD, 4, None, 0)   # opA .. act


def sk_ids():
    return [i for i, n in enumerate(sg.configs()) if n.startswith(("sk_", "sk16_"))]


def test_workspace_argument_checks():
    # misaligned, or NULL with a size: argument 16
    assert sg.sgemm_general_ws(-1, *WS_ARGS, BAD + 4, 1 << 20) == -16
    assert sg.sgemm_general_ws(-1, *WS_ARGS, None, 64) == -16
    # other arguments keep the positions of sgemm_general
    bad_lda = (0, 0, 4, 4, 8, 1.0, BAD, 7, BAD, 4, 0.0, BAD, 4, None, 0)
    assert sg.sgemm_general_ws(-1, *bad_lda, None, 0) == -8
    assert sg.sgemm_general_ws(-2, *WS_ARGS, None, 0) == sg.SGEMM_ERROR_BAD_CONFIG
    # quick return: nothing is launched and the workspace is not needed
    assert sg.sgemm_general_ws(-1, 0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None, 0, None, 0) == 0


def test_noalloc_validates_before_touching_the_device():
    """The allocation-free entry point numbers its arguments as sgemm_general and rejects
    bad ones, or returns early on an empty result, before it looks up its scratch array."""
    assert sg.sgemm_general_noalloc(-1, 0, 0, 4, 4, 8, 1.0, BAD, 7, BAD, 4, 0.0, BAD, 4, None, 0) == -8  # lda < K
    assert sg.sgemm_general_noalloc(-1, 2, *WS_ARGS[1:]) == -1
    assert sg.sgemm_general_noalloc(-1, *WS_ARGS[:14], 5) == -15                      # act
    assert sg.sgemm_general_noalloc(-2, *WS_ARGS) == sg.SGEMM_ERROR_BAD_CONFIG
    assert sg.sgemm_general_noalloc(sg.sgemm_config_count(), *WS_ARGS) == sg.SGEMM_ERROR_BAD_CONFIG
    assert sg.sgemm_general_noalloc(-1, 0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None, 0) == 0
    # the array holds the counters and two 128 x 128 partial tiles for each of 256 compute units
    assert sg.SGEMM_NOALLOC_SCRATCH_BYTES == 65536 + 2 * 256 * 128 * 128 * 4
    text = open(HEADER).read()
    assert "#define SGEMM_NOALLOC_SCRATCH_BYTES (65536ull + 2ull * 256ull * 128ull * 128ull * 4ull)" in text


def test_forced_stream_k_needs_a_workspace():
    for cid in sk_ids():
        assert sg.sgemm_general_ws(cid, *WS_ARGS, None, 0) == sg.SGEMM_ERROR_WORKSPACE
        assert sg.sgemm_general(cid, *WS_ARGS) == sg.SGEMM_ERROR_WORKSPACE
    assert "workspace" in sg.sgemm_status_string(sg.SGEMM_ERROR_WORKSPACE)


def test_workspace_size_without_a_device_is_zero():
    import ctypes
    try:
        n = ctypes.c_int(0)
        have_gpu = ctypes.CDLL("libamdhip64.so").hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0
    except OSError:
        have_gpu = False
    if not have_gpu:
        assert sg.sgemm_workspace_size(-1) == 0
    assert sg.sgemm_workspace_size(1) == 0      # data-parallel configurations need none


def test_launch_shape_stream_k():
    """Direct-copy configurations run whole rounds of 256 tiles but the last one tile per
    workgroup; the remaining tiles x K-tiles (all of them for register-staged
    configurations) are shared by 256 workgroups, or one per K-tile step when fewer."""
    for cid in sk_ids():
        name = sg.sgemm_config_name(cid)
        bm, bn, bk = (int(x) for x in name.split("_")[1].split("x"))
        for M, N, K in [(1024, 2304, 768), (100, 130, 64), (1000, 1537, 777), (4096, 4096, 256), (64, 64, 4096)]:
            tiles, iters = -(-M // bm) * -(-N // bn), -(-K // bk)
            whole = 256 * ((tiles - 1) // 256) if name.endswith("d") else 0
            st, grid, block = sg.sgemm_launch_shape(cid, M, N, K)
            assert st == 0 and grid == (whole + min(256, (tiles - whole) * iters), 1, 1), (M, N, K, grid)
            assert block[0] in (256, 512, 1024)
        # a 64 x 128 direct-copy tile's QKV layer: 288 tiles, so 256 whole and 32 shared by 256
        # workgroups; the register-staged one shares all 288 among 256
        if (bm, bn) == (64, 128):
            assert sg.sgemm_launch_shape(cid, 1024, 2304, 768)[1] == ((512 if name.endswith("d") else 256), 1, 1)


def test_select_without_workspace_never_picks_stream_k():
    names = sg.configs()
    for M, N, K in [(1024, 2304, 768), (1024, 768, 3072), (1025, 1025, 1025), (4096, 4096, 4096)]:
        assert not names[sg.sgemm_select_config(M, N, K, 1.0, BAD, K, BAD, N, BAD, N)].startswith(("sk_", "sk16_"))
        assert not names[sg.sgemm_select_config_ws(M, N, K, 1.0, BAD, K, BAD, N, BAD, N, 0)].startswith(("sk_", "sk16_"))


def test_workspace_cache_does_not_deadlock(monkeypatch):
    """workspace_for() queries the library (which takes the loader's lock) while
    filling its cache: it must not hold a lock the loader also takes. The CUDA pieces
    are stubbed so the host path runs here; a deadlock shows up as the thread never
    finishing."""
    import contextlib
    import threading
    torch = pytest.importorskip("torch")
    real_zeros = torch.zeros
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    class _Stream:                           # the current stream: fills are waited for on it
        cuda_stream = 0
        synced = 0

        def synchronize(self):
            _Stream.synced += 1
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: _Stream())
    monkeypatch.setattr(torch.cuda, "device", lambda dev: contextlib.nullcontext())
    monkeypatch.setattr(torch, "zeros", lambda *a, **k: real_zeros(*a, dtype=k.get("dtype")))
    monkeypatch.setattr(sg, "_workspaces", {})
    out = []
    th = threading.Thread(target=lambda: out.append(sg.workspace_for()), daemon=True)
    th.start()
    th.join(timeout=20)
    assert not th.is_alive(), "workspace_for() deadlocked"
    assert out and out[0].numel() >= 16 and int(out[0].sum()) == 0
    assert _Stream.synced == 1               # the zero fill is complete before the buffer is used
    assert sg.workspace_for() is out[0]      # cached
    assert _Stream.synced == 1


# sgemm_strided: M N K alpha A rsA csA B rsB csB beta C rsC csC bias act stream
_STRIDED_OK = (4, 5, 3, 1.0, BAD, 7, 2, BAD, 11, 3, 0.5, BAD, 20, 2, None, 0, None)


@pytest.mark.parametrize("pos,value,code", [
    (0, -1, -1), (1, -1, -2), (2, -1, -3),
    (4, None, -5), (5, -1, -6), (6, -2, -7), (7, None, -8), (8, -1, -9), (9, -3, -10),
    (11, None, -12), (12, -1, -13), (13, -1, -14), (15, 2, -16),
    # C windows whose entries would share addresses: rows 2 floats apart with 5 columns 2 apart
    (12, 8, -13),
    # offsets past 2^60 floats, reported at the operand's row stride
    (5, 1 << 62, -6), (9, 1 << 61, -9), (12, 1 << 60, -13),
    # a column stride of 0 for C with N > 1
    (13, 0, -13),
])
def test_strided_invalid_arguments(pos, value, code):
    args = list(_STRIDED_OK)
    args[pos] = value
    assert sg.sgemm_strided(*args) == code


def test_strided_checks_and_quick_returns():
    ok = list(_STRIDED_OK)
    # unread operands may be anything on the quick returns; M or N zero launches nothing
    assert sg.sgemm_strided(0, 5, 3, 1.0, None, -0, 0, None, 0, 0, 0.0, None, 0, 0, None, 0, None) == 0
    assert sg.sgemm_strided(4, 0, 3, 1.0, None, 0, 0, None, 0, 0, 0.0, None, 0, 0, None, 0, None) == 0
    # strides of 0 are valid for A and B (a repeated row or column); column-major C is valid
    a = [4, 5, 3, 1.0, BAD, 0, 1, BAD, 1, 0, 0.0, None, 1, 4, None, 0, None]
    assert sg.sgemm_strided(*a) == -12    # C null with M, N > 0: rejected after A's and B's strides passed
    ok[12], ok[13] = 1, 4             # column-major C (rows 1 apart, columns M = 4 apart): accepted
    ok[11] = None
    assert sg.sgemm_strided(*ok) == -12
    # M == 1 or N == 1: only the stride that walks the window must be positive
    assert sg.sgemm_strided(1, 5, 3, 1.0, BAD, 0, 0, BAD, 0, 0, 0.0, BAD, 0, 0, None, 0, None) == -14
    assert sg.sgemm_strided(4, 1, 3, 1.0, BAD, 0, 0, BAD, 0, 0, 0.0, BAD, 0, 7, None, 0, None) == -13


def test_launch_shape_fringe_columns():
    """Data-parallel matrix configurations hand the last N mod BN columns (1..8 of them) to
    workgroups of their own, two rows each, once the whole tiles number 256 or more and a
    fringe workgroup needs at most three memory round trips (its threads take 64 (NT / 64) U k
    per trip, U = 4, 2 or 1 for up to 2, 4 or 8 columns): the 1000 x 1537 x 777 product on
    64 x 64 tiles runs 16 x 24 tiles and 500 fringe workgroups. Nine columns over, too long a
    K, too few whole tiles, stream-K and the vector-ALU kernel keep the plain grid."""
    names = sg.configs()
    c64 = names.index("mfma16_64x64x32_w4x1k1d")
    assert sg.sgemm_launch_shape(c64, 1000, 1537, 777) == (0, (16 * 24 + 500, 1, 1), (256, 1, 1))
    # eight columns: one k step of 256 per round trip, so K up to 768 (three trips)
    assert sg.sgemm_launch_shape(c64, 1000, 1544, 768)[1][0] == 16 * 24 + 500
    assert sg.sgemm_launch_shape(c64, 1000, 1544, 777)[1][0] == 16 * 25       # four trips: plain tiles
    assert sg.sgemm_launch_shape(c64, 1000, 1537, 3072)[1][0] == 16 * 24 + 500
    assert sg.sgemm_launch_shape(c64, 1000, 1537, 3073)[1][0] == 16 * 25
    assert sg.sgemm_launch_shape(c64, 1000, 1545, 777)[1][0] == 16 * 25          # 9 columns over
    assert sg.sgemm_launch_shape(c64, 1000, 1536, 777)[1][0] == 16 * 24          # none over
    assert sg.sgemm_launch_shape(c64, 1000, 961, 777)[1][0] == 16 * 16           # 240 whole tiles: too few
    assert sg.sgemm_launch_shape(c64, 1023, 1025, 777)[1][0] == 16 * 16 + 512
    c32 = names.index("mfma16_32x64x64_w2x1k2d")
    assert sg.sgemm_launch_shape(c32, 1000, 1537, 777)[1][0] == 32 * 24 + 500
    # a tall product whose fringe workgroups would run in many rounds (or pass 2^32 threads)
    # keeps the plain tiles
    tall = 1 << 25
    assert sg.sgemm_launch_shape(c64, tall, 65, 64) == (0, ((tall // 64) * 2, 1, 1), (256, 1, 1))
    assert sg.sgemm_launch_shape(c64, 1 << 21, 65, 64)[1][0] == (1 << 15) * 2
    # the 256 x 256 tile holds 128 KiB of LDS, one workgroup per CU, fringe ones included: 2048
    # fringe workgroups would run in eight rounds, 256 of them in one
    big = names.index("mfma_256x256x32_w2x4d")
    assert sg.sgemm_launch_shape(big, 4096, 4100, 1024)[1][0] == 16 * 17
    assert sg.sgemm_launch_shape(big, 512, 128 * 256 + 4, 1024)[1][0] == 256 + 256
    sk = names.index("sk16_64x64x32_w4x1k1d")
    assert sg.sgemm_launch_shape(sk, 1000, 1537, 777)[1][0] == 256 + 256    # 400 tiles: 256 whole, 144 shared
    valu = names.index("valu_128x128x8_t8x8")
    assert sg.sgemm_launch_shape(valu, 1000, 1537, 777)[1][0] == 8 * 13
