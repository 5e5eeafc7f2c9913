"""Strict-FP32 SGEMM for AMD Instinct MI355X (gfx950): C = alpha*A*B + beta*C.

The computation runs in the HIP library ``libsgemm_gfx950.so`` (sources in
``csrc/``, C interface in ``include/sgemm.h``).  This package is its thin
Python binding:

* ``sgemm``, ``sgemm_ex`` and the other ``sgemm_*`` functions take exactly the
  C arguments (device pointers as ints, ``stream`` as a ``hipStream_t`` int);
* ``gemm(A, B, C, alpha, beta)`` marshals torch tensors into that call --
  shapes, leading dimensions from the row strides, data pointers and the
  current torch stream -- and raises on a non-zero status.

PyTorch only supplies device memory and streams; there is no fallback path,
and the functions raise ``LibraryMissing`` when the library is not built.
"""
from __future__ import annotations

from ._lib import (EXPORTS, LIBRARY, SGEMM_ATOMICS_ALLOWED,  # noqa: F401
                   SGEMM_ATOMICS_NOT_ALLOWED, SGEMM_ERR_DEVICE, SGEMM_ERR_DIM, SGEMM_ERR_GRID,
                   SGEMM_ERR_LAUNCH,
                   SGEMM_ERR_LD, SGEMM_ERR_OP, SGEMM_ERR_PTR, SGEMM_ERR_STRIDE,
                   SGEMM_ERR_VARIANT, SGEMM_NO_KERNEL, SGEMM_OK, SGEMM_OP_N, SGEMM_OP_T,
                   LibraryMissing, load, sgemm, sgemm_ceiling_copy, sgemm_ceiling_empty,
                   sgemm_ceiling_fma, sgemm_ceiling_mfma, sgemm_ceiling_read, sgemm_ex,
                   sgemm_get_atomics_mode, sgemm_num_variants, sgemm_op, sgemm_op_ex,
                   sgemm_op_select_variant, sgemm_select_variant, sgemm_set_atomics_mode,
                   sgemm_status_string, sgemm_strided_batched, sgemm_strided_batched_ex,
                   sgemm_strided_batched_select_variant, sgemm_strided_batched_ws,
                   sgemm_strided_batched_ws_ex, sgemm_strided_batched_ws_select_variant,
                   sgemm_variant_name, sgemm_version, sgemm_workspace_size, SGEMM_ERR_WORKSPACE,
                   sgemm_strided_batched_noalloc)

__all__ = ["gemm", "gemm_batched", "variant_names", "sgemm", "sgemm_ex", "sgemm_op",
           "sgemm_op_ex", "sgemm_op_select_variant", "sgemm_strided_batched",
           "sgemm_strided_batched_ex", "sgemm_strided_batched_select_variant", "sgemm_num_variants",
           "sgemm_strided_batched_ws", "sgemm_strided_batched_ws_ex",
           "sgemm_strided_batched_ws_select_variant", "sgemm_workspace_size", "workspace",
           "sgemm_strided_batched_noalloc",
           "sgemm_variant_name", "sgemm_select_variant", "sgemm_status_string",
           "sgemm_version", "sgemm_set_atomics_mode", "sgemm_get_atomics_mode",
           "sgemm_ceiling_mfma", "sgemm_ceiling_fma", "sgemm_ceiling_copy",
           "sgemm_ceiling_read", "sgemm_ceiling_empty",
           "LibraryMissing", "SgemmError"]


class SgemmError(RuntimeError):
    """A non-zero status from the C library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__("sgemm status %d: %s" % (status, sgemm_status_string(status)))


def variant_names():
    return [sgemm_variant_name(i) for i in range(sgemm_num_variants())]


def _leading_dim(t, rows, cols, name):
    """Leading dimension of a 2-D float32 tensor used as a row-major matrix.

    Every row must be contiguous (unit column stride) whenever a row holds
    more than one element, whatever the number of rows: a one-row view with a
    column stride would otherwise be read or written as if it were packed."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if tuple(t.shape) != (rows, cols):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (rows, cols)))
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major (stride(1) == 1)" % name)
    if rows <= 1:
        return max(1, cols)
    return t.stride(0)


def _same_hip_device(A, B, C):
    for name, t in (("A", A), ("B", B), ("C", C)):
        if not t.is_cuda:
            raise ValueError("%s must be on a HIP device" % name)
    if len({t.device for t in (A, B, C)}) != 1:
        raise ValueError("A, B and C must be on the same device")


def workspace(M: int, N: int, K: int, *, trans_a: bool = False, trans_b: bool = False,
              device=None):
    """A zero-filled device buffer of the size ``sgemm_workspace_size``
    gives for this problem (a uint8 tensor), or None when the problem has
    no use for one.  Allocated by torch; reusable for later calls."""
    import torch
    n = sgemm_workspace_size(SGEMM_OP_T if trans_a else SGEMM_OP_N,
                             SGEMM_OP_T if trans_b else SGEMM_OP_N, M, N, K, 1)
    if n < 0:
        raise SgemmError(n)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, *, trans_a: bool = False,
         trans_b: bool = False, variant: int = -1, stream=None, workspace=None):
    """C = alpha * op(A) @ op(B) + beta * C in place on float32 HIP tensors;
    returns C.

    op(A) is A (M x K) or, with trans_a, the transpose of the K x M tensor A;
    op(B) is B (K x N) or, with trans_b, the transpose of the N x K tensor B.
    Every tensor is row-major (unit column stride; the row stride is the
    leading dimension).  The call is enqueued on ``stream`` (default: the
    current torch stream) and does not synchronise.  ``workspace``: an
    optional zero-filled device tensor (see ``workspace()``) that lets the
    call split its last partial round of tiles (sgemm_strided_batched_ws)."""
    import torch
    M = int(A.shape[1] if trans_a else A.shape[0])
    K = int(A.shape[0] if trans_a else A.shape[1])
    N = int(B.shape[0] if trans_b else B.shape[1])
    kb = int(B.shape[1] if trans_b else B.shape[0])
    if kb != K:
        raise ValueError("inner dimensions differ: op(A) has K=%d, op(B) has K=%d" % (K, kb))
    lda = _leading_dim(A, K if trans_a else M, M if trans_a else K, "A")
    ldb = _leading_dim(B, N if trans_b else K, K if trans_b else N, "B")
    ldc = _leading_dim(C, M, N, "C")
    _same_hip_device(A, B, C)
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    opa = SGEMM_OP_T if trans_a else SGEMM_OP_N
    opb = SGEMM_OP_T if trans_b else SGEMM_OP_N
    with torch.cuda.device(C.device):
        if workspace is None:
            st = sgemm_op_ex(opa, opb, M, N, K, float(alpha), A.data_ptr() or None, lda,
                             B.data_ptr() or None, ldb, float(beta), C.data_ptr() or None, ldc,
                             handle, variant)
        else:
            if not workspace.is_cuda or workspace.device != C.device:
                raise ValueError("workspace must be on C's device")
            nbytes = workspace.numel() * workspace.element_size()
            st = sgemm_strided_batched_ws_ex(opa, opb, M, N, K, float(alpha), A.data_ptr() or None,
                                             lda, 0, B.data_ptr() or None, ldb, 0, float(beta),
                                             C.data_ptr() or None, ldc, 0, 1, workspace.data_ptr(),
                                             nbytes, handle, variant)
    if st != SGEMM_OK:
        raise SgemmError(st)
    return C


def _batch_stride(t, name):
    if t.dim() != 3:
        raise ValueError("%s must be 3-D (batch, rows, cols)" % name)
    return t.stride(0) if t.shape[0] > 1 else 0


def gemm_batched(A, B, C, alpha: float = 1.0, beta: float = 0.0, *, trans_a: bool = False,
                 trans_b: bool = False, variant: int = -1, stream=None):
    """C[z] = alpha * op(A[z]) @ op(B[z]) + beta * C[z] for every z, in place on
    3-D float32 HIP tensors (batch, rows, cols), each slice row-major; returns
    C.  A or B may be broadcast along the batch (stride 0, e.g. from
    ``expand``).  One strided-batched call, enqueued on ``stream``."""
    import torch
    if not (A.dim() == B.dim() == C.dim() == 3):
        raise ValueError("A, B and C must be 3-D")
    batch = int(C.shape[0])
    if A.shape[0] != batch or B.shape[0] != batch:
        raise ValueError("batch sizes differ: %d, %d, %d" % (A.shape[0], B.shape[0], batch))
    if batch == 0:
        return C
    a0, b0, c0 = A[0], B[0], C[0]
    M = int(a0.shape[1] if trans_a else a0.shape[0])
    K = int(a0.shape[0] if trans_a else a0.shape[1])
    N = int(b0.shape[0] if trans_b else b0.shape[1])
    kb = int(b0.shape[1] if trans_b else b0.shape[0])
    if kb != K:
        raise ValueError("inner dimensions differ: op(A) has K=%d, op(B) has K=%d" % (K, kb))
    lda = _leading_dim(a0, K if trans_a else M, M if trans_a else K, "A")
    ldb = _leading_dim(b0, N if trans_b else K, K if trans_b else N, "B")
    ldc = _leading_dim(c0, M, N, "C")
    _same_hip_device(A, B, C)
    sa, sb, sc = A.stride(0), B.stride(0), C.stride(0)
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(C.device):
        st = sgemm_strided_batched_ex(
            SGEMM_OP_T if trans_a else SGEMM_OP_N, SGEMM_OP_T if trans_b else SGEMM_OP_N, M, N, K,
            float(alpha), A.data_ptr() or None, lda, sa, B.data_ptr() or None, ldb, sb, float(beta),
            C.data_ptr() or None, ldc, sc, batch, handle, variant)
    if st != SGEMM_OK:
        raise SgemmError(st)
    return C
