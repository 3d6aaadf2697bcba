"""The direct-copy LDS layouts, checked on the host with the kernels' own index functions.

``layout_check`` (built from ``csrc/layout_check.hip``) walks every direct-copy
configuration in all four operand forms and both copy widths. It checks that each copy
instruction lands its data where the layout says, that the copies cover the tile exactly
once, that the layout is one-to-one, and that the matrix-core loop's fragment reads meet
no bank conflict in a model of the 64-bank LDS. No GPU is needed: only host code runs.
"""

import subprocess


def test_direct_copy_layouts():
    from tiled_fp32_gemm_02_amd import build as sgbuild
    exe = sgbuild.ensure_layout_check()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout, res.stdout
