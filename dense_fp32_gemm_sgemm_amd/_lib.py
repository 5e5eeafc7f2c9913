"""ctypes binding of ``libsgemm_gfx950.so`` -- argument marshalling only.

Every function here has the name and arguments of the C entry point it wraps
(declared in ``include/sgemm.h`` and ``include/sgemm_ceiling.h``): sizes and
scalars are passed through, matrices are device pointers given as Python ints,
and ``stream`` is a ``hipStream_t`` as an int (0 = default stream).  No step of
the computation runs in Python, and there is no fallback: if the library is
missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsgemm_gfx950.so")

SGEMM_OK = 0
SGEMM_ERR_DIM = -1
SGEMM_ERR_LD = -2
SGEMM_ERR_PTR = -3
SGEMM_ERR_LAUNCH = -4
SGEMM_ERR_DEVICE = -5
SGEMM_ERR_VARIANT = -6
SGEMM_ERR_OP = -7
SGEMM_ERR_STRIDE = -8
SGEMM_ERR_GRID = -9
SGEMM_ERR_WORKSPACE = -10
SGEMM_NO_KERNEL = -100
SGEMM_OP_N = 0
SGEMM_OP_T = 1
SGEMM_ATOMICS_NOT_ALLOWED = 0
SGEMM_ATOMICS_ALLOWED = 1

# Every exported symbol, as declared in include/*.h.
EXPORTS = ("sgemm", "sgemm_ex", "sgemm_op", "sgemm_op_ex", "sgemm_strided_batched",
           "sgemm_strided_batched_ex", "sgemm_num_variants", "sgemm_variant_name",
           "sgemm_select_variant", "sgemm_op_select_variant", "sgemm_strided_batched_select_variant",
           "sgemm_status_string", "sgemm_version", "sgemm_set_atomics_mode",
           "sgemm_get_atomics_mode", "sgemm_strided_batched_ws", "sgemm_strided_batched_ws_ex",
           "sgemm_strided_batched_ws_select_variant", "sgemm_workspace_size",
           "sgemm_strided_batched_noalloc",
           "sgemm_ceiling_mfma", "sgemm_ceiling_fma", "sgemm_ceiling_copy", "sgemm_ceiling_read",
           "sgemm_ceiling_empty")

_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    """The HIP library has not been built (run ``__graft_entry__.build()``)."""


def _declare(lib):
    c_int, c_float, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    gemm_args = [c_int, c_int, c_int, c_float, vp, c_int, vp, c_int, c_float, vp, c_int, vp]
    lib.sgemm.argtypes = gemm_args
    lib.sgemm.restype = c_int
    lib.sgemm_ex.argtypes = gemm_args + [c_int]
    lib.sgemm_ex.restype = c_int
    lib.sgemm_op.argtypes = [c_int, c_int] + gemm_args
    lib.sgemm_op.restype = c_int
    lib.sgemm_op_ex.argtypes = [c_int, c_int] + gemm_args + [c_int]
    lib.sgemm_op_ex.restype = c_int
    lib.sgemm_op_select_variant.argtypes = [c_int, c_int, c_int, c_int, c_int, c_float, vp, c_int,
                                            vp, c_int, c_float, vp, c_int]
    lib.sgemm_op_select_variant.restype = c_int
    i64 = ctypes.c_longlong
    batched = [c_int, c_int, c_int, c_int, c_int, c_float, vp, c_int, i64, vp, c_int, i64, c_float,
               vp, c_int, i64, c_int]
    lib.sgemm_strided_batched.argtypes = batched + [vp]
    lib.sgemm_strided_batched.restype = c_int
    lib.sgemm_strided_batched_ex.argtypes = batched + [vp, c_int]
    lib.sgemm_strided_batched_ex.restype = c_int
    lib.sgemm_strided_batched_select_variant.argtypes = batched
    lib.sgemm_strided_batched_select_variant.restype = c_int
    u64 = ctypes.c_ulonglong
    lib.sgemm_strided_batched_ws.argtypes = batched + [vp, u64, vp]
    lib.sgemm_strided_batched_ws.restype = c_int
    lib.sgemm_strided_batched_ws_ex.argtypes = batched + [vp, u64, vp, c_int]
    lib.sgemm_strided_batched_ws_ex.restype = c_int
    lib.sgemm_strided_batched_ws_select_variant.argtypes = batched + [u64]
    lib.sgemm_strided_batched_ws_select_variant.restype = c_int
    lib.sgemm_strided_batched_noalloc.argtypes = batched + [vp]
    lib.sgemm_strided_batched_noalloc.restype = c_int
    lib.sgemm_workspace_size.argtypes = [c_int] * 6
    lib.sgemm_workspace_size.restype = ctypes.c_longlong
    lib.sgemm_num_variants.argtypes = []
    lib.sgemm_num_variants.restype = c_int
    lib.sgemm_variant_name.argtypes = [c_int]
    lib.sgemm_variant_name.restype = ctypes.c_char_p
    lib.sgemm_select_variant.argtypes = [c_int, c_int, c_int, c_float, vp, c_int, vp, c_int,
                                         c_float, vp, c_int]
    lib.sgemm_select_variant.restype = c_int
    lib.sgemm_status_string.argtypes = [c_int]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_version.argtypes = []
    lib.sgemm_version.restype = c_int
    lib.sgemm_set_atomics_mode.argtypes = [c_int]
    lib.sgemm_set_atomics_mode.restype = c_int
    lib.sgemm_get_atomics_mode.argtypes = []
    lib.sgemm_get_atomics_mode.restype = c_int
    dp = ctypes.POINTER(ctypes.c_double)
    lib.sgemm_ceiling_mfma.argtypes = [c_int, c_int, c_int, vp, vp, dp]
    lib.sgemm_ceiling_mfma.restype = c_int
    lib.sgemm_ceiling_fma.argtypes = [c_int, c_int, vp, vp, dp]
    lib.sgemm_ceiling_fma.restype = c_int
    lib.sgemm_ceiling_copy.argtypes = [vp, vp, ctypes.c_longlong, c_int, vp]
    lib.sgemm_ceiling_copy.restype = c_int
    lib.sgemm_ceiling_read.argtypes = [vp, ctypes.c_longlong, c_int, vp, vp]
    lib.sgemm_ceiling_read.restype = c_int
    lib.sgemm_ceiling_empty.argtypes = [c_int, vp]
    lib.sgemm_ceiling_empty.restype = c_int
    return lib


def load():
    """The loaded library; raises LibraryMissing if it was never built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise LibraryMissing(
                    "%s not found: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                    % LIBRARY)
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C = alpha*A*B + beta*C on ``stream``; returns the C status code."""
    return load().sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, variant=-1) -> int:
    """As ``sgemm`` with an explicit kernel variant (-1 = automatic)."""
    return load().sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def sgemm_op(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C = alpha*op(A)*op(B) + beta*C; op is SGEMM_OP_N or SGEMM_OP_T."""
    return load().sgemm_op(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_op_ex(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
                variant=-1) -> int:
    return load().sgemm_op_ex(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                              variant)


def sgemm_op_select_variant(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    return load().sgemm_op_select_variant(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


def sgemm_strided_batched(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                          ldc, strideC, batch, stream=0) -> int:
    """C_z = alpha*op(A_z)*op(B_z) + beta*C_z for z < batch (element strides)."""
    return load().sgemm_strided_batched(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
                                        beta, C, ldc, strideC, batch, stream)


def sgemm_strided_batched_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                             ldc, strideC, batch, stream=0, variant=-1) -> int:
    return load().sgemm_strided_batched_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                           strideB, beta, C, ldc, strideC, batch, stream, variant)


def sgemm_strided_batched_select_variant(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                         strideB, beta, C, ldc, strideC, batch) -> int:
    return load().sgemm_strided_batched_select_variant(opA, opB, M, N, K, alpha, A, lda, strideA,
                                                       B, ldb, strideB, beta, C, ldc, strideC,
                                                       batch)


def sgemm_strided_batched_ws(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                             ldc, strideC, batch, workspace, workspace_bytes, stream=0) -> int:
    """sgemm_strided_batched with a caller workspace (device pointer, bytes)."""
    return load().sgemm_strided_batched_ws(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                           strideB, beta, C, ldc, strideC, batch, workspace,
                                           workspace_bytes, stream)


def sgemm_strided_batched_ws_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta,
                                C, ldc, strideC, batch, workspace, workspace_bytes, stream=0,
                                variant=-1) -> int:
    return load().sgemm_strided_batched_ws_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                              strideB, beta, C, ldc, strideC, batch, workspace,
                                              workspace_bytes, stream, variant)


def sgemm_strided_batched_ws_select_variant(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                            strideB, beta, C, ldc, strideC, batch,
                                            workspace_bytes) -> int:
    return load().sgemm_strided_batched_ws_select_variant(opA, opB, M, N, K, alpha, A, lda,
                                                          strideA, B, ldb, strideB, beta, C, ldc,
                                                          strideC, batch, workspace_bytes)


def sgemm_strided_batched_noalloc(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta,
                                  C, ldc, strideC, batch, stream=0) -> int:
    """sgemm_strided_batched_ws on the library's static scratch (allocates nothing)."""
    return load().sgemm_strided_batched_noalloc(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                                strideB, beta, C, ldc, strideC, batch, stream)


def sgemm_workspace_size(opA, opB, M, N, K, batch=1) -> int:
    return load().sgemm_workspace_size(opA, opB, M, N, K, batch)


def sgemm_num_variants() -> int:
    return load().sgemm_num_variants()


def sgemm_variant_name(variant: int) -> str:
    return load().sgemm_variant_name(variant).decode()


def sgemm_select_variant(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    return load().sgemm_select_variant(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


def sgemm_status_string(status: int) -> str:
    return load().sgemm_status_string(status).decode()


def sgemm_version() -> int:
    return load().sgemm_version()


def sgemm_set_atomics_mode(mode) -> int:
    """SGEMM_ATOMICS_ALLOWED or SGEMM_ATOMICS_NOT_ALLOWED (process-wide)."""
    return load().sgemm_set_atomics_mode(mode)


def sgemm_get_atomics_mode() -> int:
    return load().sgemm_get_atomics_mode()


def sgemm_ceiling_mfma(shape, blocks, iters, sink, stream=0):
    """Returns (status, flops of the launch)."""
    flops = ctypes.c_double(0.0)
    st = load().sgemm_ceiling_mfma(shape, blocks, iters, sink, stream, ctypes.byref(flops))
    return st, flops.value


def sgemm_ceiling_fma(blocks, iters, sink, stream=0):
    """Returns (status, flops of the launch)."""
    flops = ctypes.c_double(0.0)
    st = load().sgemm_ceiling_fma(blocks, iters, sink, stream, ctypes.byref(flops))
    return st, flops.value


def sgemm_ceiling_copy(src, dst, n, blocks, stream=0) -> int:
    return load().sgemm_ceiling_copy(src, dst, n, blocks, stream)


def sgemm_ceiling_read(src, n, blocks, sink, stream=0) -> int:
    return load().sgemm_ceiling_read(src, n, blocks, sink, stream)


def sgemm_ceiling_empty(blocks, stream=0) -> int:
    return load().sgemm_ceiling_empty(blocks, stream)
