"""Every kernel compiles for gfx950 with the resources its launch assumes (CPU only).

Checks, from the compiler's own kernel metadata for our device code:
  - no private (scratch) memory and no register spills in any kernel;
  - LDS per workgroup within gfx950's 160 KiB;
  - the VGPR+AGPR count fits the waves a workgroup puts on each SIMD
    (512 registers per lane per SIMD, waves spread over 4 SIMDs);
  - the matrix kernels really issue the fp32 matrix instruction.
The GPT-2 post assembles device code on GPU-less CI machines so malformed code
fails before it reaches hardware ("GPU Target", section "NVVM to PTX"); this is
the same idea for our gfx950 build.
"""

import os
import re
import subprocess

import pytest
import yaml

from tiled_fp32_gemm_02_amd import build as sgbuild

LDS_LIMIT = 160 * 1024


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    path = str(tmp_path_factory.mktemp("asm") / "sgemm.s")
    sgbuild.device_asm(path)
    text = open(path).read()
    out = {}
    for block in re.findall(r"\.amdgpu_metadata\n(.*?)\.end_amdgpu_metadata", text, re.S):
        meta = yaml.safe_load(block.replace("\t", "  "))
        for k in meta["amdhsa.kernels"]:
            name = k[".name"]
            # the whole function, up to its end label (a kernel can end in several places)
            body = re.search(r"^" + re.escape(name) + r":[^\n]*\n(.*?)^\.Lfunc_end\d+:", text, re.S | re.M).group(1)
            demangled = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
            out[demangled] = (k, body)
    return out


def parse_config(name):
    m = re.fullmatch(r"(mfma|mfma16|sk|sk16)_(\d+)x(\d+)x(\d+)_w(\d+)x(\d+)(?:k(\d+))?(?:p(\d+))?(d)?", name)
    assert m, name
    bm, bn, bk, wm, wn = (int(x) for x in m.groups()[1:6])
    mb = 16 if m.group(1) in ("mfma16", "sk16") else 32
    return bm, bn, bk, wm, wn, int(m.group(7) or 1), int(m.group(8) or 1), m.group(9) is not None, mb


def expected_mfma_kernels(config_names):
    """Template arguments <BM,BN,BK,WGM,WGN,WGK,PF,DMA,TA,TB,VEC,EDGE> of every matrix
    kernel the launcher can start: per configuration and operand form, the aligned
    whole-tile and edge variants as configured; for register-staged configurations
    (stream-K ones included) the unaligned variant with their own K-tile and loads in
    flight; for direct-copy ones the register-staged unaligned variant with one K-tile in
    flight and K-tiles of 16 * WGK (row strides the direct copies cannot take), and the
    unaligned variant of the direct copies (16-byte copies from 4-byte aligned rows, the
    K-tile holding the end of K in 4-byte words) with the configured K-tiles in flight."""
    out = set()
    for name in config_names:
        bm, bn, bk, wm, wn, wk, pf, dma, mb = parse_config(name)
        nt = wm * wn * wk * 64
        for ta in (0, 1):
            for tb in (0, 1):
                if name.startswith("mfma"):
                    for edge in (0, 1):
                        out.add((bm, bn, bk, wm, wn, wk, pf, int(dma), ta, tb, 1, edge, mb))
                    if dma:
                        out.add((bm, bn, bk, wm, wn, wk, pf, 1, ta, tb, 0, 1, mb))
                    if dma:     # two k groups per wave group: 16 k (32x32 blocks) or 32 k (16x16 blocks)
                        out.add((bm, bn, (512 // mb) * wk, wm, wn, wk, 1, 0, ta, tb, 0, 1, mb))
                    else:
                        out.add((bm, bn, bk, wm, wn, wk, pf, 0, ta, tb, 0, 1, mb))
                else:
                    # stream-K: the register-staged tile kernel for operands it cannot take (unaligned
                    # ones of a register-staged configuration, or row strides direct copies cannot take)
                    out.add((bm, bn, bk, wm, wn, wk, pf, 0, ta, tb, 0, 1, mb))
    return out


def expected_sk_kernels(config_names):
    """Stream-K kernels: the aligned whole-tile and edge variants of each stream-K
    configuration, and for direct-copy ones the unaligned variant of the direct copies
    (register-staged configurations run the data-parallel kernel of the tile on unaligned
    operands)."""
    out = set()
    for name in config_names:
        bm, bn, bk, wm, wn, wk, pf, dma, mb = parse_config(name)
        nt = wm * wn * wk * 64
        for ta in (0, 1):
            for tb in (0, 1):
                for edge in (0, 1):
                    out.add((bm, bn, bk, wm, wn, wk, pf, int(dma), ta, tb, 1, edge, mb))
                if dma:
                    out.add((bm, bn, bk, wm, wn, wk, pf, 1, ta, tb, 0, 1, mb))
    return out


def test_all_kernels_present(kernels):
    names = " ".join(kernels)
    assert "sgemm_tile16" in names and "sgemm_scale" in names and "sgemm_valu" in names
    import tiled_fp32_gemm_02_amd as sg
    names = [n for n in sg.configs() if n.startswith(("mfma_", "mfma16_", "sk_", "sk16_"))]
    for kind, expected in (("sgemm_mfma", expected_mfma_kernels(names)),
                           ("sgemm_mfma_sk", expected_sk_kernels([c for c in names if c.startswith(("sk_", "sk16_"))]))):
        found = set()
        for n in kernels:
            m = re.search(kind + r"<([^>]*)>", n)
            if m:
                found.add(tuple(int(x) if x.strip().lstrip("-").isdigit() else int(x.strip() == "true")
                                for x in m.group(1).split(",")))
        assert found == expected, kind


def test_no_scratch_no_spills(kernels):
    for name, (k, _) in kernels.items():
        assert k[".private_segment_fixed_size"] == 0, name
        assert k[".vgpr_spill_count"] == 0 and k[".sgpr_spill_count"] == 0, name


def test_lds_within_limit(kernels):
    for name, (k, _) in kernels.items():
        assert k[".group_segment_fixed_size"] <= LDS_LIMIT, name


def test_registers_fit_the_launch(kernels):
    for name, (k, _) in kernels.items():
        threads = k[".max_flat_workgroup_size"]
        waves_per_simd = -(-(threads // 64) // 4)
        assert k[".vgpr_count"] <= 512 // waves_per_simd, (name, k[".vgpr_count"], threads)


def test_matrix_kernels_use_fp32_mfma(kernels):
    """Each matrix kernel issues the fp32 instruction of its block size (the last template
    argument): v_mfma_f32_32x32x2_f32 for 32, v_mfma_f32_16x16x4_f32 for 16, and not the other."""
    sizes = set()
    for name, (k, body) in kernels.items():
        m = re.search(r"sgemm_mfma(?:_sk)?<[^>]*, (\d+)>", name)
        if m:
            mb = int(m.group(1))
            sizes.add(mb)
            want, other = ("v_mfma_f32_16x16x4_f32", "v_mfma_f32_32x32x2_f32") if mb == 16 else \
                ("v_mfma_f32_32x32x2_f32", "v_mfma_f32_16x16x4_f32")
            assert want in body and other not in body, name
    assert sizes == {16, 32}


def test_vector_kernel_uses_plain_fma(kernels):
    """The micro-tile reference runs on the vector ALU: fused multiply-adds, no matrix
    instructions and no packed fp32 forms (the build keeps those off)."""
    found = 0
    for name, (k, body) in kernels.items():
        if "sgemm_valu<" in name:
            found += 1
            assert "v_fma_f32" in body or "v_fmac_f32" in body, name
            assert "v_mfma" not in body and "v_pk_fma_f32" not in body and "v_pk_mul_f32" not in body, name
    assert found == 4


def test_oracle_builds():
    import oracle
    path = oracle.build(force=True)
    assert os.path.exists(path)
