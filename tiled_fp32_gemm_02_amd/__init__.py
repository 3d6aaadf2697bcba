"""Python binding of the MI355X fp32 GEMM library (``libsgemm.so``).

Argument marshalling only: every entry point here forwards to the C function of
the same name in ``include/sgemm.h``; all arithmetic runs in the library's HIP
kernels. PyTorch supplies device memory and streams. There is no CPU fallback:
if the library is missing or fails to load, every call raises.

Raw entry points take device addresses as Python ints (or CUDA tensors, whose
``data_ptr()`` is used) and return the library's status code:

    sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    sgemm_ex(config, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    sgemm_op(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    sgemm_bias_act(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream)
    sgemm_general(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream)
    sgemm_general_ws(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                     workspace, workspace_bytes, stream)
    sgemm_general_noalloc(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream)
    sgemm_strided_batched(M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch, stream)
    sgemm_strided_batched_op(opA, opB, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch, stream)
    sgemm_strided_batched_general(config, opA, opB, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC,
                                  bias, act, batch, stream)

``gemm(A, B, C=None, alpha=1, beta=0, bias=None, act=None)`` is the tensor-level
form: it checks shapes, dtypes and devices, reads a transposed view (unit row
stride) as a transposed operand in place, fills in the leading dimensions from the
tensors' strides, raises ``ValueError``/``RuntimeError`` on bad input or a nonzero
status, and returns C. By default it passes a workspace (one zero-filled buffer per
device and stream, made once with PyTorch) so that the library may pick its stream-K
configurations; ``workspace=None`` keeps to the data-parallel ones.
"""

from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "load", "lib_path", "sgemm", "sgemm_ex", "sgemm_strided_batched", "sgemm_config_count",
    "sgemm_config_name", "sgemm_config_describe", "describe", "sgemm_select_config", "sgemm_launch_shape",
    "sgemm_status_string",
    "sgemm_version", "sgemm_op", "sgemm_bias_act", "sgemm_general", "configs", "gemm", "gemm_batched",
    "check", "SgemmError", "SGEMM_ERROR_TOO_LARGE", "SGEMM_ERROR_BAD_CONFIG", "SGEMM_OP_N", "SGEMM_OP_T",
    "SGEMM_ACT_NONE", "SGEMM_ACT_GELU_TANH", "SGEMM_ERROR_WORKSPACE", "sgemm_general_ws", "sgemm_workspace_size",
    "sgemm_select_config_ws", "workspace_for", "sgemm_strided_batched_op", "sgemm_strided_batched_general",
    "sgemm_select_config_general", "sgemm_general_noalloc", "SGEMM_NOALLOC_SCRATCH_BYTES", "sgemm_strided",
]

SGEMM_ERROR_TOO_LARGE = -100
SGEMM_ERROR_BAD_CONFIG = -101
SGEMM_ERROR_WORKSPACE = -102
SGEMM_OP_N = 0
SGEMM_OP_T = 1
SGEMM_ACT_NONE = 0
SGEMM_ACT_GELU_TANH = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsgemm.so")
_lock = threading.Lock()
_lib = None

_fp = ctypes.c_void_p
_SIGS = {
    "sgemm": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int,
                             _fp, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, _fp]),
    "sgemm_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp,
                                ctypes.c_int, _fp, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, _fp]),
    "sgemm_op": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int, ctypes.c_float, _fp,
                                ctypes.c_int, _fp]),
    "sgemm_bias_act": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int, ctypes.c_float,
                                      _fp, ctypes.c_int, _fp, ctypes.c_int, _fp]),
    "sgemm_general": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int,
                                     ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int, _fp]),
    "sgemm_general_ws": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int,
                                        ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int, _fp,
                                        ctypes.c_size_t, _fp]),
    "sgemm_general_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int,
                                             ctypes.c_float, _fp, ctypes.c_int, _fp, ctypes.c_int, _fp]),
    "sgemm_strided": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_longlong, ctypes.c_longlong,
        _fp, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_float, _fp, ctypes.c_longlong, ctypes.c_longlong,
        _fp, ctypes.c_int, _fp]),
    "sgemm_workspace_size": (ctypes.c_size_t, [ctypes.c_int]),
    "sgemm_select_config_ws": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp,
                                              ctypes.c_int, _fp, ctypes.c_int, _fp, ctypes.c_int, ctypes.c_size_t]),
    "sgemm_strided_batched": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int, ctypes.c_longlong,
        _fp, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, _fp, ctypes.c_int, ctypes.c_longlong,
        ctypes.c_int, _fp]),
    "sgemm_strided_batched_op": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int,
        ctypes.c_longlong, _fp, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, _fp, ctypes.c_int,
        ctypes.c_longlong, ctypes.c_int, _fp]),
    "sgemm_strided_batched_general": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp,
        ctypes.c_int, ctypes.c_longlong, _fp, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, _fp, ctypes.c_int,
        ctypes.c_longlong, _fp, ctypes.c_int, ctypes.c_int, _fp]),
    "sgemm_select_config_general": (ctypes.c_int, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp, ctypes.c_int,
        ctypes.c_longlong, _fp, ctypes.c_int, ctypes.c_longlong, _fp, ctypes.c_int, ctypes.c_longlong,
        ctypes.c_int, ctypes.c_size_t]),
    "sgemm_config_count": (ctypes.c_int, []),
    "sgemm_config_name": (ctypes.c_char_p, [ctypes.c_int]),
    "sgemm_config_describe": (ctypes.c_char_p, [ctypes.c_int]),
    "sgemm_select_config": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, _fp,
                                           ctypes.c_int, _fp, ctypes.c_int, _fp, ctypes.c_int]),
    "sgemm_launch_shape": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
    "sgemm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sgemm_version": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


class SgemmError(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, status: int, what: str = "sgemm"):
        self.status = status
        super().__init__(f"{what}: status {status}: {sgemm_status_string(status)}")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libsgemm.so (once). Raises RuntimeError if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build the HIP library first "
                    "(python -m tiled_fp32_gemm_02_amd.build, or __graft_entry__.build())")
            lib = ctypes.CDLL(_LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _addr(x):
    """Device address of a tensor or int (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


# --------------------------------------------------------------------------- raw C-ABI forms

def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return load().sgemm(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc, _stream(stream))


def sgemm_ex(config, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return load().sgemm_ex(config, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                           _stream(stream))


def sgemm_op(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return load().sgemm_op(opA, opB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                           _stream(stream))


def sgemm_bias_act(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream=None) -> int:
    return load().sgemm_bias_act(opA, opB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                                 _addr(bias), act, _stream(stream))


def sgemm_general(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream=None) -> int:
    return load().sgemm_general(config, opA, opB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C),
                                ldc, _addr(bias), act, _stream(stream))


def sgemm_general_ws(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, workspace,
                     workspace_bytes, stream=None) -> int:
    return load().sgemm_general_ws(config, opA, opB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                   _addr(C), ldc, _addr(bias), act, _addr(workspace), workspace_bytes,
                                   _stream(stream))


def sgemm_general_noalloc(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                          stream=None) -> int:
    return load().sgemm_general_noalloc(config, opA, opB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                        _addr(C), ldc, _addr(bias), act, _stream(stream))


SGEMM_NOALLOC_SCRATCH_BYTES = 65536 + 2 * 256 * 128 * 128 * 4


def sgemm_strided(M, N, K, alpha, A, rsA, csA, B, rsB, csB, beta, C, rsC, csC, bias=None, act=SGEMM_ACT_NONE,
                  stream=None) -> int:
    return load().sgemm_strided(M, N, K, alpha, _addr(A), rsA, csA, _addr(B), rsB, csB, beta, _addr(C), rsC, csC,
                                _addr(bias), act, _stream(stream))


def sgemm_workspace_size(config: int = -1) -> int:
    return load().sgemm_workspace_size(config)


def sgemm_select_config_ws(M, N, K, alpha, A, lda, B, ldb, C, ldc, workspace_bytes) -> int:
    return load().sgemm_select_config_ws(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                                         workspace_bytes)


def sgemm_strided_batched(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                          batch, stream=None) -> int:
    return load().sgemm_strided_batched(M, N, K, alpha, _addr(A), lda, strideA, _addr(B), ldb, strideB,
                                        beta, _addr(C), ldc, strideC, batch, _stream(stream))


def sgemm_strided_batched_op(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                             batch, stream=None) -> int:
    return load().sgemm_strided_batched_op(opA, opB, M, N, K, alpha, _addr(A), lda, strideA, _addr(B), ldb,
                                           strideB, beta, _addr(C), ldc, strideC, batch, _stream(stream))


def sgemm_strided_batched_general(config, opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                                  ldc, strideC, bias, act, batch, stream=None) -> int:
    return load().sgemm_strided_batched_general(config, opA, opB, M, N, K, alpha, _addr(A), lda, strideA,
                                                _addr(B), ldb, strideB, beta, _addr(C), ldc, strideC, _addr(bias),
                                                act, batch, _stream(stream))


def sgemm_select_config_general(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                                batch, workspace_bytes=0) -> int:
    return load().sgemm_select_config_general(opA, opB, M, N, K, alpha, _addr(A), lda, strideA, _addr(B), ldb,
                                              strideB, _addr(C), ldc, strideC, batch, workspace_bytes)


def sgemm_config_count() -> int:
    return load().sgemm_config_count()


def sgemm_config_name(config: int):
    name = load().sgemm_config_name(config)
    return name.decode() if name is not None else None


def sgemm_config_describe(config: int):
    line = load().sgemm_config_describe(config)
    return line.decode() if line is not None else None


def describe(config: int) -> dict:
    """The fields of sgemm_config_describe(config) as a dict (ValueError if out of range)."""
    line = sgemm_config_describe(config)
    if line is None:
        raise ValueError(f"no configuration {config}")
    return dict(field.split("=", 1) for field in line.split())


def sgemm_select_config(M, N, K, alpha, A, lda, B, ldb, C, ldc) -> int:
    return load().sgemm_select_config(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, _addr(C), ldc)


def sgemm_launch_shape(config, M, N, K):
    """Returns (status, grid, block)."""
    grid = (ctypes.c_int * 3)()
    block = (ctypes.c_int * 3)()
    st = load().sgemm_launch_shape(config, M, N, K, grid, block)
    return st, tuple(grid), tuple(block)


def sgemm_status_string(status: int) -> str:
    return load().sgemm_status_string(status).decode()


def sgemm_version() -> str:
    return load().sgemm_version().decode()


def configs():
    """List of configuration names, indexed by id."""
    return [sgemm_config_name(i) for i in range(sgemm_config_count())]


def check(status: int, what: str = "sgemm") -> None:
    if status != 0:
        raise SgemmError(status, what)


# --------------------------------------------------------------------------- tensor form

def _check_matrix(t, name):
    if t.dim() != 2:
        raise ValueError(f"Dimension error: {name} must be a 2-D matrix, got {t.dim()} dimensions")
    if str(t.dtype) != "torch.float32":
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _stored_form(t):
    """(op, ld) when an operand view is a stored row-major matrix read as stored
    (SGEMM_OP_N: unit column stride, row stride at least the row length) or in place as a
    transpose (SGEMM_OP_T: unit row stride, column stride at least the column length);
    None for any other layout (no unit stride, or rows that overlap in memory)."""
    rows, cols = t.shape
    s0, s1 = t.stride()
    if cols <= 1 or s1 == 1:
        if rows <= 1:
            return SGEMM_OP_N, max(cols, 1)
        if s0 >= max(cols, 1):
            return SGEMM_OP_N, s0
    if rows <= 1 or s0 == 1:
        if cols <= 1:
            return SGEMM_OP_T, max(rows, 1)
        if s1 >= max(rows, 1):
            return SGEMM_OP_T, s1
    return None


def _row_major_c(t):
    """ldc when C is a row-major view whose rows do not overlap; None otherwise."""
    form = _stored_form(t)
    rows, cols = t.shape
    if form is None or (form[0] == SGEMM_OP_T and cols > 1):
        return None
    return form[1] if rows > 1 else max(cols, 1)


_ACTS = {None: SGEMM_ACT_NONE, "none": SGEMM_ACT_NONE, "gelu_tanh": SGEMM_ACT_GELU_TANH}
_workspaces = {}
_ws_lock = threading.Lock()      # guards _workspaces only; never held while calling the library


def workspace_for(device=None, stream=None):
    """The stream-K workspace for (device, stream): a zero-filled uint8 GPU tensor of
    sgemm_workspace_size() bytes, made once and reused. Calls on one stream run in
    order, so they can share it; each stream gets its own.

    The zero fill is queued on the device's current stream, which need not be
    `stream`; the fill is waited for before the buffer is handed out, so the first
    launch on `stream` (or on any stream) cannot overtake it."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev.index, _stream(stream))
    with _ws_lock:
        ws = _workspaces.get(key)
    if ws is not None:
        return ws
    with torch.cuda.device(dev):
        nbytes = sgemm_workspace_size(-1)   # loads the library: not under _ws_lock
        fresh = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
        torch.cuda.current_stream(dev).synchronize()
    with _ws_lock:
        return _workspaces.setdefault(key, fresh)


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, stream=None, config: int = -1, bias=None,
         act=None, workspace="auto"):
    """C <- act(alpha*A@B + beta*C + bias) on GPU float32 tensors.

    A is M x K, B is K x N and C is M x N, any strided views (slices, transposes, expanded
    dimensions for A and B), read and written in place. Row-major views and transposed
    views of row-major matrices run the stored-matrix kernels (with stream-K where the
    workspace allows); other layouts run the general-stride entry point, sgemm_strided
    (then config must be -1). bias is a length-N float32 GPU vector or None; act is
    None, "none" or "gelu_tanh". When C is None a new M x N tensor is allocated (then
    beta must be 0). workspace is "auto" (the cached buffer of ``workspace_for()`` for
    this device and stream), None (no stream-K), or a zero-initialised uint8 GPU tensor
    of the caller's. Returns C.
    """
    import torch

    _check_matrix(A, "A")
    _check_matrix(B, "B")
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError(f"Size error: A is {tuple(A.shape)} and B is {tuple(B.shape)}; inner sizes differ")
    N = B.shape[1]
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(k for k in _ACTS if k)} or None, got {act!r}")
    if bias is not None:
        if bias.dim() != 1 or bias.shape[0] != N or str(bias.dtype) != "torch.float32" or not bias.is_cuda:
            raise ValueError(f"bias must be a float32 GPU vector of length {N}")
        if bias.stride(0) != 1 and N > 1:
            raise ValueError("bias must be contiguous")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check_matrix(C, "C")
    if tuple(C.shape) != (M, N):
        raise ValueError(f"Size error: C is {tuple(C.shape)}, expected {(M, N)}")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    fa, fb, ldc = _stored_form(A), _stored_form(B), _row_major_c(C)
    if fa is None or fb is None or ldc is None:
        if config != -1:
            raise ValueError("config applies to row-major or transposed views only; this layout runs sgemm_strided")
        check(sgemm_strided(M, N, K, alpha, A, A.stride(0), A.stride(1), B, B.stride(0), B.stride(1), beta, C,
                            C.stride(0), C.stride(1), bias, _ACTS[act], stream), "sgemm_strided")
        return C
    (opA, lda), (opB, ldb) = fa, fb
    ws = workspace_for(A.device, stream) if isinstance(workspace, str) and workspace == "auto" else workspace
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(sgemm_general_ws(config, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, _ACTS[act],
                           ws, nbytes, stream), "sgemm_general_ws")
    return C


def _batched_operand(t, name, allow_transposed=True):
    """(op, ld, batch stride) of a batch x rows x cols view. The last two dimensions are
    read as for gemm(): unit column stride -> as stored, unit row stride -> a transpose
    read in place (only if allow_transposed)."""
    if t.dim() != 3:
        raise ValueError(f"Dimension error: {name} must be 3-D (batch, rows, cols), got {t.dim()} dimensions")
    if str(t.dtype) != "torch.float32":
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    bsz, rows, cols = t.shape
    s0, s1, s2 = t.stride()
    sb = s0 if bsz > 1 else 0
    if (cols <= 1 or s2 == 1) and (rows <= 1 or s1 >= cols):
        ld = s1 if rows > 1 else max(cols, 1)
        return SGEMM_OP_N, max(ld, cols, 1), sb
    if allow_transposed and (rows <= 1 or s1 == 1) and (cols <= 1 or s2 >= rows):
        ld = s2 if cols > 1 else max(rows, 1)
        return SGEMM_OP_T, max(ld, rows, 1), sb
    what = ("a unit stride in one of its last two dimensions, rows that do not overlap" if allow_transposed
            else "unit column stride and rows that do not overlap")
    raise ValueError(f"{name} needs {what} (got strides {tuple(t.stride())})")


def gemm_batched(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, stream=None, config: int = -1, bias=None,
                 act=None):
    """Batched C[b] <- act(alpha*A[b]@B[b] + beta*C[b] + bias) on 3-D GPU float32 tensors.

    Each operand is batch x rows x cols. A and B may be views whose last two dimensions
    are row-major or transposed (``x.transpose(1, 2)``), read in place; C needs unit
    column stride. The batch and row strides come from the tensors, so per-head views of
    one matrix (e.g. ``qkv[:, :768].view(T, 12, 64).transpose(0, 1)``) need no copies,
    and C may be heads side by side in one matrix. bias (length N, shared by all
    batches) and act as for gemm(). Returns C.
    """
    import torch

    opA, lda, sA = _batched_operand(A, "A")
    opB, ldb, sB = _batched_operand(B, "B")
    bsz, M, K = A.shape
    if B.shape[0] != bsz or B.shape[1] != K:
        raise ValueError(f"Size error: A is {tuple(A.shape)} and B is {tuple(B.shape)}")
    N = B.shape[2]
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(k for k in _ACTS if k)} or None, got {act!r}")
    if bias is not None:
        if bias.dim() != 1 or bias.shape[0] != N or str(bias.dtype) != "torch.float32" or not bias.is_cuda:
            raise ValueError(f"bias must be a float32 GPU vector of length {N}")
        if bias.stride(0) != 1 and N > 1:
            raise ValueError("bias must be contiguous")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((bsz, M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (bsz, M, N):
        raise ValueError(f"Size error: C is {tuple(C.shape)}, expected {(bsz, M, N)}")
    _, ldc, sC = _batched_operand(C, "C", allow_transposed=False)
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    check(sgemm_strided_batched_general(config, opA, opB, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc,
                                        sC, bias, _ACTS[act], bsz, stream), "sgemm_strided_batched_general")
    return C
