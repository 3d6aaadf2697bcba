"""CPU oracle for row-major fp32 GEMM, C = alpha*A*B + beta*C.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``. The GPU library
and its Python binding never import it, and it shares no code with them.

The arithmetic lives in ``sgemm_oracle.c`` (plain C, fp64 accumulation, compiled
with gcc, no fast-math, no FP contraction). This module only loads it and
marshals numpy arrays. ``exact.py`` holds an exact rational brute force for
tiny problems. ``within_bound`` applies the pass criterion:

    |c_gpu - ref| <= bound   elementwise,   bound = 4*max(K,1)*2^-24*(|alpha|*g + |beta*c0|)

where g is the sum of |a_ik * b_kj|. The accepted error covers any fp32
summation order and any use of fused multiply-add; the GPT-2 post ("GPU
Target", section "Running it") attributes tiled-versus-library differences to
the order of accumulation, which is why the comparison is not bitwise.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = ["sgemm", "sgemm_entries", "gemm", "gemm_entries", "gelu_tanh", "within_bound", "threads",
           "build", "LIB_PATH", "ACT_NONE", "ACT_GELU_TANH"]

ACT_NONE = 0
ACT_GELU_TANH = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "sgemm_oracle.c")
LIB_PATH = os.path.join(_HERE, "libsgemm_oracle.so")
_lock = threading.Lock()
_lib = None

_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no FP contraction)."""
    if not force and os.path.exists(LIB_PATH) and os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH):
        return LIB_PATH
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-fPIC", "-shared", SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(LIB_PATH)
            lib.oracle_threads.restype = ctypes.c_int
            lib.oracle_sgemm_f64.restype = ctypes.c_int
            lib.oracle_sgemm_f64.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                _F32P, ctypes.c_int64, _F32P, ctypes.c_int64,
                ctypes.c_float, _F32P, ctypes.c_int64,
                _F64P, ctypes.c_int64, _F64P, ctypes.c_int64]
            lib.oracle_sgemm_entries_f64.restype = ctypes.c_int
            lib.oracle_sgemm_entries_f64.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                _F32P, ctypes.c_int64, _F32P, ctypes.c_int64,
                ctypes.c_float, _F32P, ctypes.c_int64,
                ctypes.c_int64, _I64P, _I64P, _F64P, _F64P]
            lib.oracle_gemm_f64.restype = ctypes.c_int
            lib.oracle_gemm_f64.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                _F32P, ctypes.c_int64, _F32P, ctypes.c_int64,
                ctypes.c_float, _F32P, ctypes.c_int64, _F32P, ctypes.c_int,
                _F64P, ctypes.c_int64, _F64P, ctypes.c_int64]
            lib.oracle_gemm_entries_f64.restype = ctypes.c_int
            lib.oracle_gemm_entries_f64.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                _F32P, ctypes.c_int64, _F32P, ctypes.c_int64,
                ctypes.c_float, _F32P, ctypes.c_int64, _F32P, ctypes.c_int,
                ctypes.c_int64, _I64P, _I64P, _F64P, _F64P]
            lib.oracle_gelu_tanh.restype = ctypes.c_double
            lib.oracle_gelu_tanh.argtypes = [ctypes.c_double]
            _lib = lib
    return _lib


def threads() -> int:
    """Host threads the oracle uses (OpenMP over rows of C)."""
    return int(_load().oracle_threads())


def _fptr(x, need_rows, ld, cols, name):
    """Pointer to a C-contiguous float32 buffer holding `need_rows` rows of stride `ld`."""
    if need_rows == 0 or cols == 0:
        return ctypes.cast(None, _F32P), None
    arr = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    need = (need_rows - 1) * ld + cols
    if arr.size < need:
        raise ValueError(f"{name}: buffer holds {arr.size} floats, needs {need}")
    return arr.ctypes.data_as(_F32P), arr


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, *, with_bound=True):
    """Oracle result for the M x N window: returns (ref, bound) as float64 arrays.

    A, B, C are float32 buffers read row-major with leading dimensions lda, ldb,
    ldc (C only when beta != 0; pass None otherwise). `bound` is None when
    ``with_bound`` is False.
    """
    lib = _load()
    nonempty = M > 0 and N > 0
    use_ab = nonempty and alpha != 0.0 and K > 0
    pa, ka = _fptr(A, M if use_ab else 0, lda, K, "A")
    pb, kb = _fptr(B, K if use_ab else 0, ldb, N, "B")
    pc, kc = _fptr(C, M if (nonempty and beta != 0.0) else 0, ldc, N, "C")
    ref = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = lib.oracle_sgemm_f64(
        M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
        ref.ctypes.data_as(_F64P), N,
        bound.ctypes.data_as(_F64P) if with_bound else ctypes.cast(None, _F64P), N)
    if rc != 0:
        raise MemoryError("oracle_sgemm_f64 could not allocate its row buffers")
    del ka, kb, kc
    return ref, bound


def sgemm_entries(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols):
    """Oracle (ref, bound) for the sampled entries (rows[e], cols[e]) only."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same shape")
    nonempty = M > 0 and N > 0 and rows.size > 0
    use_ab = nonempty and alpha != 0.0 and K > 0
    pa, ka = _fptr(A, M if use_ab else 0, lda, K, "A")
    pb, kb = _fptr(B, K if use_ab else 0, ldb, N, "B")
    pc, kc = _fptr(C, M if (nonempty and beta != 0.0) else 0, ldc, N, "C")
    ref = np.empty(rows.shape, dtype=np.float64)
    bound = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_sgemm_entries_f64(
        M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
        rows.size, rows.ctypes.data_as(_I64P), cols.ctypes.data_as(_I64P),
        ref.ctypes.data_as(_F64P), bound.ctypes.data_as(_F64P))
    if rc != 0:
        raise IndexError("sampled entry outside the M x N result")
    del ka, kb, kc
    return ref, bound


def _operand_rows(op, rows_as_read, cols_as_read):
    """Stored (rows, cols) of an operand read as rows_as_read x cols_as_read under op."""
    return (cols_as_read, rows_as_read) if op else (rows_as_read, cols_as_read)


def gemm(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias=None, act=ACT_NONE, *,
         with_bound=True):
    """Oracle (ref, bound) for act(alpha * op(A) op(B) + beta * C + bias) on the M x N window.

    op == 0 reads an operand as stored, op == 1 its transpose (A stored K x M, B stored
    N x K, row-major with leading dimension lda / ldb). bias has N entries (by column) or
    is None; act is ACT_NONE or ACT_GELU_TANH.
    """
    lib = _load()
    nonempty = M > 0 and N > 0
    use_ab = nonempty and alpha != 0.0 and K > 0
    ar, ac = _operand_rows(opA, M, K)
    br, bc = _operand_rows(opB, K, N)
    pa, ka = _fptr(A, ar if use_ab else 0, lda, ac, "A")
    pb, kb = _fptr(B, br if use_ab else 0, ldb, bc, "B")
    pc, kc = _fptr(C, M if (nonempty and beta != 0.0) else 0, ldc, N, "C")
    pbias, kbias = _fptr(bias, 1 if (nonempty and bias is not None) else 0, N, N, "bias")
    ref = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = lib.oracle_gemm_f64(
        int(opA), int(opB), M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc, pbias, int(act),
        ref.ctypes.data_as(_F64P), N,
        bound.ctypes.data_as(_F64P) if with_bound else ctypes.cast(None, _F64P), N)
    if rc == -2:
        raise ValueError("op must be 0 or 1 and act must be ACT_NONE or ACT_GELU_TANH")
    if rc != 0:
        raise MemoryError("oracle_gemm_f64 could not allocate its row buffers")
    del ka, kb, kc, kbias
    return ref, bound


def gemm_entries(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols, bias=None,
                 act=ACT_NONE):
    """Oracle (ref, bound) for the sampled entries (rows[e], cols[e]) of ``gemm``."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same shape")
    nonempty = M > 0 and N > 0 and rows.size > 0
    use_ab = nonempty and alpha != 0.0 and K > 0
    ar, ac = _operand_rows(opA, M, K)
    br, bc = _operand_rows(opB, K, N)
    pa, ka = _fptr(A, ar if use_ab else 0, lda, ac, "A")
    pb, kb = _fptr(B, br if use_ab else 0, ldb, bc, "B")
    pc, kc = _fptr(C, M if (nonempty and beta != 0.0) else 0, ldc, N, "C")
    pbias, kbias = _fptr(bias, 1 if (nonempty and bias is not None) else 0, N, N, "bias")
    ref = np.empty(rows.shape, dtype=np.float64)
    bound = np.empty(rows.shape, dtype=np.float64)
    rc = lib.oracle_gemm_entries_f64(
        int(opA), int(opB), M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc, pbias, int(act),
        rows.size, rows.ctypes.data_as(_I64P), cols.ctypes.data_as(_I64P),
        ref.ctypes.data_as(_F64P), bound.ctypes.data_as(_F64P))
    if rc == -2:
        raise ValueError("op must be 0 or 1 and act must be ACT_NONE or ACT_GELU_TANH")
    if rc != 0:
        raise IndexError("sampled entry outside the M x N result")
    del ka, kb, kc, kbias
    return ref, bound


def gelu_tanh(x: float) -> float:
    """The oracle's fp64 tanh-form GELU, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return float(_load().oracle_gelu_tanh(float(x)))


def within_bound(c, ref, bound):
    """Apply the pass criterion. Returns (ok, max_ratio, argmax_index).

    ``c`` holds the fp32 results being checked (any shape matching ref). The
    ratio is |c - ref| / bound (0/0 counts as 0; a NaN anywhere fails).
    """
    c64 = np.asarray(c, dtype=np.float64)
    err = np.abs(c64 - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(err == 0.0, 0.0, err / bound)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    if ratio.size == 0:
        return True, 0.0, None
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    worst = float(ratio[idx])
    return bool(worst <= 1.0), worst, idx
