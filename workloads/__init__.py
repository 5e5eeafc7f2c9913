"""Seeded synthetic inputs for the SGEMM checks and benchmark.

This module holds no GEMM arithmetic: it only draws matrices.  Both the oracle
side (tests, CPU baseline) and the GPU side (tests, benchmark) take their
inputs from here, so the two always see the same bits.

The pages never state a value distribution or print a matrix: every workload on
them is a random dense square matrix, and the benchmark in "The road to a fast
GEMM" (section "The complete code") fills its inputs from a seeded helper that
is not shown.  The plainest reading is used here:

  * real inputs: A, B i.i.d. uniform on [-1, 1]; C (when beta != 0) i.i.d.
    standard normal; all drawn in float64 by ``numpy.random.default_rng(seed)``
    in the order A, B, C and rounded to float32;
  * exact-check copies: A, B (and C) i.i.d. uniform integers in {-4, ..., 4},
    for which every partial sum of a K <= 2^19 dot product stays an integer
    below 2^24 and is therefore exact in fp32;
  * A != B (they are separate draws).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Square sizes of the sweep and the ragged / rectangular shapes.
SWEEP_SIZES = (128, 256, 512, 1024, 2048, 4096, 8192)
RAGGED_SHAPES = ((4095, 4097, 1023), (8192, 1024, 8192), (1024, 8192, 256),
                 (127, 129, 17), (1, 4096, 4096))
# One GPU's share of the 4096^3 problem split over eight GPUs: by rows of C
# (each GPU holds 512 rows of A and all of B) and on a 2 x 4 grid of C blocks.
SHARD_SHAPES = ((512, 4096, 4096), (2048, 1024, 4096))


@dataclass(frozen=True)
class Workload:
    """One GEMM problem: shape, scalars, value kind and seed."""
    name: str
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    kind: str = "real"          # "real" or "int"
    seed: int = 0
    notes: str = field(default="", compare=False)


# The small case, the headline case and the accumulate case, plus their
# exact-check copies.
SMALL = Workload("square-256", 256, 256, 256, 1.0, 0.0, "real", 0)
SMALL_INT = Workload("square-256-int", 256, 256, 256, 1.0, 0.0, "int", 0)
HEADLINE = Workload("square-4096", 4096, 4096, 4096, 1.0, 0.0, "real", 0)
ACCUM = Workload("square-4096-accumulate", 4096, 4096, 4096, 1.5, 0.5, "real", 0)
ACCUM_INT = Workload("square-4096-accumulate-int", 4096, 4096, 4096, 1.0, 1.0, "int", 0)


def sweep_workloads():
    return [Workload("square-%d" % n, n, n, n, 1.0, 0.0, "real", n) for n in SWEEP_SIZES]


def shard_workloads():
    return [Workload("shard-%dx%dx%d" % s, s[0], s[1], s[2], 1.0, 0.0, "real", 200 + i)
            for i, s in enumerate(SHARD_SHAPES)]


def ragged_workloads():
    return [Workload("shape-%dx%dx%d" % s, s[0], s[1], s[2], 1.0, 0.0, "real", 100 + i)
            for i, s in enumerate(RAGGED_SHAPES)]


def draw(M: int, N: int, K: int, *, seed: int, kind: str = "real",
         with_c: bool = False):
    """(A, B, C) as contiguous float32 arrays; C is None unless ``with_c``."""
    rng = np.random.default_rng(seed)
    if kind == "real":
        A = rng.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
        B = rng.uniform(-1.0, 1.0, (K, N)).astype(np.float32)
        C = rng.standard_normal((M, N)).astype(np.float32) if with_c else None
    elif kind == "int":
        A = rng.integers(-4, 5, (M, K)).astype(np.float32)
        B = rng.integers(-4, 5, (K, N)).astype(np.float32)
        C = rng.integers(-4, 5, (M, N)).astype(np.float32) if with_c else None
    else:
        raise ValueError("kind must be 'real' or 'int'")
    return A, B, C


def draw_workload(w: Workload):
    """Inputs for a named workload (C drawn only when beta != 0)."""
    return draw(w.M, w.N, w.K, seed=w.seed, kind=w.kind, with_c=(w.beta != 0.0))


def padded(X: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Copy X (rows x cols) into a buffer with leading dimension ``ld``,
    filling the gap columns with ``fill``; returns the (rows x cols) view."""
    rows, cols = X.shape
    if ld < cols:
        raise ValueError("ld %d < cols %d" % (ld, cols))
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = X
    return buf[:, :cols]


def offset_view(X: np.ndarray, offset_elems: int, ld: int | None = None,
                fill: float = np.nan) -> np.ndarray:
    """Copy X into a buffer so that its first element sits ``offset_elems``
    floats past a 64-byte boundary (misaligned when offset % 4 != 0)."""
    rows, cols = X.shape
    ld = cols if ld is None else ld
    total = offset_elems + (rows - 1) * ld + cols if rows else offset_elems
    raw = np.full(total + 16, fill, dtype=np.float32)
    shift = (-(raw.ctypes.data // 4)) % 16
    base = raw[shift:shift + total]
    flat = base[offset_elems:]
    view = np.lib.stride_tricks.as_strided(flat, shape=(rows, cols), strides=(ld * 4, 4))
    view[...] = X
    return view
