"""Build the HIP library ``libsgemm.so`` in-tree for gfx950.

One translation unit (``csrc/sgemm_api.hip``, which includes the kernels) is
compiled by hipcc into a shared library next to this file. Flags:

* ``--offload-arch=gfx950``: MI355X only; no other targets, no CUDA.
* ``-O3 -std=c++17 -fPIC -shared``.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: keep the compiler from
  emitting packed fp32 VALU instructions. The GEMM's arithmetic runs on the
  matrix cores; the packed forms are not trusted on the target machines.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "sgemm_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "sgemm_kernels.hpp"), os.path.join(INCLUDE, "sgemm.h")]
LIB_PATH = os.path.join(HERE, "libsgemm.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile libsgemm.so (always recompiles). Returns its path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), *COMMON_FLAGS, "-fPIC", "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of the library's device code (for resource checks)."""
    cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", *SOURCES, "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out_path


def ensure_built() -> str:
    """Build only if no library exists yet (tests, smoke and bench call this)."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
