"""CPU oracle for single-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and the
oracle shares no code with it: the arithmetic lives in ``sgemm_oracle.c`` (plain
C, fp64 accumulation, OpenMP over output rows), and this module only marshals
numpy arrays into it and compares results.

Definition followed (see ``sgemm_oracle.c`` for the full statement): with A of
size MxK, B of size KxN and C of size MxN, all row-major FP32,

    C_ref = alpha * (A @ B) + beta * C_in

("The road to a fast GEMM", section "The problem and the ceiling"; each element
is the dot product of a row of A and a column of B, "Optimizing SGEMM in CUDA",
section "What is a SGEMM?").  Sums and products are taken in double.

Acceptance rules for a GPU result C (fp32):
  * ``exact_match``: C converted to double equals C_ref element by element
    (used on small-integer inputs, where every partial sum is an integer below
    2^24 and so exactly representable in fp32);
  * ``normalized_error``: max |C - C_ref| / D with
    D = sum_k |A_ik||B_kj| + |beta C_ij|, which must be <= 1e-5; where D == 0
    the result must be exactly 0.

Parity status: pinned -- every function here is checked in
``tests/test_oracle.py`` against exact rational arithmetic, brute force over
all tiny {-1,0,1} problems, closed forms, identity / permutation / rank-1
structure, and a float64 library matmul; planted-mistake builds of the C file
must each fail at least one of those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sgemm_oracle.c")
LIBRARY = os.path.join(_HERE, "libsgemm_oracle.so")

_lock = threading.Lock()
_lib = None


def build(output: str = LIBRARY, source: str = SOURCE, quiet: bool = True) -> str:
    """Compile ``sgemm_oracle.c`` (or, for the planted-mistake tests, an
    altered copy given as ``source``) with gcc into a shared library."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           source, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stderr)
    os.replace(tmp, output)
    if not quiet:
        print(" ".join(cmd))
    return output


def _declare(lib):
    i64, dbl = ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    for name in ("oracle_sgemm_rows", "oracle_sgemm_cols"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64,
                       vp, i64, vp, vp]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if it is missing).

    With ``path`` given, loads that file (used for planted-mistake builds)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY) or (
                    os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
                build()
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle's row loop uses."""
    return int(load().oracle_max_threads())


def _matrix_args(X, rows, cols, name):
    """(pointer, leading dimension) of a row-major fp32 matrix view."""
    if X is None:
        return None, max(1, cols)
    if not isinstance(X, np.ndarray) or X.dtype != np.float32 or X.ndim != 2:
        raise TypeError("%s must be a 2-D float32 numpy array" % name)
    if X.shape != (rows, cols):
        raise ValueError("%s has shape %s, expected %s" % (name, X.shape, (rows, cols)))
    if X.size == 0:
        return None, max(1, cols)
    if X.strides[1] != 4 or X.strides[0] % 4 != 0:
        raise ValueError("%s must be row-major with unit column stride" % name)
    ld = X.strides[0] // 4 if rows > 1 else max(1, cols)
    if rows > 1 and ld < cols:
        raise ValueError("%s leading dimension %d < %d" % (name, ld, cols))
    return X.ctypes.data, ld


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, *, rows=None,
         cols=None, lib=None):
    """Reference C_ref and tolerance denominator D, both float64.

    A: (M,K) float32, B: (K,N) float32, C: (M,N) float32 or None (needs
    beta == 0).  Views into larger buffers are fine: the leading dimension is
    read from the row stride and gap elements are never touched.

    ``rows``: optional sequence of output rows -> results have shape
    (len(rows), N).  ``cols``: optional sequence of output columns -> results
    have shape (M, len(cols)).  At most one of the two may be given."""
    lib = lib or load()
    M, K = A.shape if A is not None else (C.shape[0], 0)
    N = B.shape[1] if B is not None else C.shape[1]
    if B is not None and B.shape[0] != K:
        raise ValueError("inner dimensions differ: A %s, B %s" % (A.shape, B.shape))
    if beta != 0.0 and C is None:
        raise ValueError("beta != 0 needs C")
    pa, lda = _matrix_args(A, M, K, "A")
    pb, ldb = _matrix_args(B, K, N, "B")
    pc, ldc = _matrix_args(C, M, N, "C") if C is not None else (None, max(1, N))
    if rows is not None and cols is not None:
        raise ValueError("give rows or cols, not both")
    if cols is not None:
        sel = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        if sel.size and (sel.min() < 0 or sel.max() >= N):
            raise IndexError("column index out of range")
        ref = np.zeros((M, sel.size), np.float64)
        den = np.zeros((M, sel.size), np.float64)
        rc = lib.oracle_sgemm_cols(M, N, K, float(alpha), pa, lda, pb, ldb,
                                   float(beta), pc, ldc, sel.ctypes.data, sel.size,
                                   ref.ctypes.data, den.ctypes.data)
    else:
        if rows is not None:
            sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            if sel.size and (sel.min() < 0 or sel.max() >= M):
                raise IndexError("row index out of range")
            psel, nsel = sel.ctypes.data, sel.size
        else:
            sel, psel, nsel = None, None, M
        ref = np.zeros((nsel, N), np.float64)
        den = np.zeros((nsel, N), np.float64)
        rc = lib.oracle_sgemm_rows(M, N, K, float(alpha), pa, lda, pb, ldb,
                                   float(beta), pc, ldc, psel, nsel,
                                   ref.ctypes.data, den.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return ref, den


def exact_match(C, ref) -> bool:
    """True when every element of the fp32 result equals C_ref exactly
    (compared as numbers, so -0 == +0)."""
    C64 = np.asarray(C, dtype=np.float64)
    return C64.shape == ref.shape and bool(np.all(C64 == ref))


def normalized_error(C, ref, den) -> float:
    """max |C - C_ref| / D over all elements.

    Elements with D == 0 must be exactly 0 in C: any other value there (or any
    NaN where C_ref is finite) makes the error infinite."""
    C64 = np.asarray(C, dtype=np.float64)
    if C64.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (C64.shape, ref.shape))
    if C64.size == 0:
        return 0.0
    diff = np.abs(C64 - ref)
    zero = den == 0
    if np.any(zero & (C64 != 0)):
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(zero, 0.0, diff / np.where(zero, 1.0, den))
    if np.any(np.isnan(q)):
        return float("inf")
    return float(q.max())
