"""Build the HIP library ``libsgemm.so`` in-tree for gfx950.

Translation units, compiled in parallel by hipcc and linked into one shared
library next to this file:

* ``csrc/sgemm_api.hip``: the C ABI, the 16x16 baseline kernel and the scale kernel;
* ``csrc/sgemm_inst.hip`` four times, once per operand form (SGEMM_TA, SGEMM_TB),
  each instantiating every MFMA configuration of ``csrc/sgemm_configs.inc``.

It also builds two standalone executables, no part of the library:

* ``mfma_rate`` measures the fp32 matrix-core rate and the shader clock the chip
  sustains (a ceiling to read the GEMM's timings against);
* ``layout_check`` checks on the host, without a GPU, the LDS layouts of the
  direct-copy kernels with the kernels' own index functions: every copy lands where
  the layout puts its data, the tile is covered once, and the fragment reads are free
  of bank conflicts in a model of the LDS.

Flags:

* ``--offload-arch=gfx950``: MI355X only; no other targets, no CUDA.
* ``-O3 -std=c++17 -fPIC``.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: keep the compiler from
  emitting packed fp32 VALU instructions. The GEMM's arithmetic runs on the
  matrix cores; the packed forms are not trusted on the target machines.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libsgemm.so")
RATE_PATH = os.path.join(HERE, "mfma_rate")
LAYOUT_CHECK_PATH = os.path.join(HERE, "layout_check")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# (source, extra defines, object stem)
UNITS = [("sgemm_api.hip", [], "api")] + [
    ("sgemm_inst.hip", [f"-DSGEMM_TA={ta}", f"-DSGEMM_TB={tb}"], f"inst_{'t' if ta else 'n'}{'t' if tb else 'n'}")
    for ta in (0, 1) for tb in (0, 1)
]
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                 if f.endswith((".hip", ".hpp", ".inc")))


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _jobs() -> int:
    return max(1, min(len(UNITS) + 2, os.cpu_count() or 1, int(os.environ.get("MAX_JOBS", "16"))))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd)}")
    return res


def build(verbose: bool = False) -> str:
    """Compile libsgemm.so (always recompiles). Returns its path."""
    with tempfile.TemporaryDirectory(prefix="sgemm_build_") as tmpdir:
        objs = []
        cmds = []
        for src, defs, stem in UNITS:
            obj = os.path.join(tmpdir, stem + ".o")
            objs.append(obj)
            cmds.append([hipcc(), *COMMON_FLAGS, "-fPIC", *defs, "-c", os.path.join(CSRC, src), "-o", obj])
        rate_tmp = RATE_PATH + f".tmp{os.getpid()}"
        cmds.append([hipcc(), *COMMON_FLAGS, os.path.join(CSRC, "mfma_rate.hip"), "-o", rate_tmp])
        check_tmp = LAYOUT_CHECK_PATH + f".tmp{os.getpid()}"
        cmds.append(_layout_check_cmd(check_tmp))
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            list(pool.map(lambda c: _run(c, verbose), cmds))
        os.replace(rate_tmp, RATE_PATH)
        os.replace(check_tmp, LAYOUT_CHECK_PATH)
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of all device code (the units' .s files, concatenated)."""
    with tempfile.TemporaryDirectory(prefix="sgemm_asm_") as tmpdir:
        cmds, outs = [], []
        for src, defs, stem in UNITS:
            out = os.path.join(tmpdir, stem + ".s")
            outs.append(out)
            cmds.append([hipcc(), *COMMON_FLAGS, *defs, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                         "-o", out])
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            list(pool.map(lambda c: _run(c, False), cmds))
        with open(out_path, "w") as f:
            for out in outs:
                f.write(open(out).read())
                f.write("\n")
    return out_path


def _layout_check_cmd(out):
    return [hipcc(), *COMMON_FLAGS, os.path.join(CSRC, "layout_check.hip"), "-o", out]


def ensure_layout_check() -> str:
    """Build layout_check if it is missing or older than any kernel source."""
    if not os.path.exists(LAYOUT_CHECK_PATH) or \
            os.path.getmtime(LAYOUT_CHECK_PATH) < max(os.path.getmtime(f) for f in SOURCES):
        tmp = LAYOUT_CHECK_PATH + f".tmp{os.getpid()}"
        _run(_layout_check_cmd(tmp), False)
        os.replace(tmp, LAYOUT_CHECK_PATH)
    return LAYOUT_CHECK_PATH


def ensure_built() -> str:
    """Build only if no library exists yet (tests, smoke and bench call this)."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
