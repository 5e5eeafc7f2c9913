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


# Shapes (M, N, K, op(A)op(B)) on which every scored tile family is timed to
# fit and check the automatic tile choice: tile counts just past whole
# rounds, M just past a multiple of 64, few rows with a long K, mid-size
# squares, one GPU's share of a split 4096^3, and a last round left partial.
TILE_CHOICE_SHAPES = (
    (4095, 4097, 1023, "NN"), (4096, 4096, 1023, "NN"), (4096, 4097, 1024, "NN"),
    (4095, 4097, 4095, "NN"), (2047, 2049, 2047, "NN"), (8191, 1025, 8191, "NN"),
    (4096, 4096, 1024, "NN"), (1023, 8193, 257, "NN"), (2047, 4097, 4095, "NN"),
    (3000, 3000, 3000, "NN"), (3072, 3072, 3072, "NN"), (6144, 1024, 4096, "NN"),
    (2048, 2048, 512, "NN"), (10000, 10000, 1000, "NN"), (5000, 5000, 5000, "NN"),
    (3584, 3584, 3584, "NN"), (2560, 2560, 2560, "NN"), (1536, 1536, 1536, "NN"),
    (96, 16384, 4096, "NN"), (256, 16384, 4096, "NN"), (448, 4096, 8192, "NN"),
    (192, 16384, 4096, "NN"), (4095, 4097, 1023, "NT"), (4095, 4097, 1023, "TN"),
    (4095, 4097, 1023, "TT"), (96, 8192, 8192, "NN"), (96, 4096, 4096, "NN"),
    (96, 2048, 8192, "NN"), (192, 8192, 8192, "NN"), (320, 8192, 8192, "NN"),
    (320, 4096, 4096, "NN"), (384, 4096, 4096, "NN"), (1024, 1536, 8192, "NN"),
    (1536, 1024, 4096, "NN"), (512, 512, 512, "NN"), (1024, 1024, 1024, "NN"),
    (256, 4096, 4096, "NN"), (160, 4096, 4096, "NN"), (352, 8192, 8192, "NN"),
    (48, 16384, 4096, "NN"), (128, 8192, 8192, "NN"), (4096, 4096, 4096, "NN"),
    (768, 768, 768, "NN"), (1000, 1000, 1000, "NN"), (48, 8192, 8192, "NN"),
    (48, 4096, 4096, "NN"), (40, 16384, 4096, "NN"), (56, 8192, 8192, "NN"),
    (33, 8192, 8192, "NN"), (64, 8192, 8192, "NN"), (48, 4096, 16384, "NN"),
    (64, 4096, 4096, "NN"), (40, 4096, 4096, "NN"), (48, 2048, 8192, "NN"),
    (64, 2048, 8192, "NN"), (36, 1024, 8192, "NN"), (64, 4096, 16384, "NN"),
    (48, 1024, 4096, "NN"), (64, 1024, 4096, "NN"), (200, 300, 2048, "NN"),
    (96, 700, 2048, "NN"), (64, 700, 2048, "NN"), (200, 700, 2048, "NN"),
    (300, 1000, 1024, "NN"), (128, 1024, 1024, "NN"), (256, 512, 1024, "NN"),
    (128, 2048, 1024, "NN"), (512, 256, 1024, "NN"), (200, 1500, 1024, "NN"),
    (128, 1024, 1536, "NN"), (300, 1000, 1536, "NN"), (1500, 3000, 2000, "NN"),
    (700, 5000, 3000, "NN"), (3000, 700, 5000, "NN"), (2500, 2500, 1500, "NN"),
    (6000, 3000, 1000, "NN"), (1200, 1200, 8000, "NN"), (800, 9000, 2000, "NN"),
    (5000, 1500, 3000, "NN"), (384, 6000, 6000, "NN"), (2200, 4400, 700, "NN"),
    (512, 4096, 4096, "NN"), (2048, 1024, 4096, "NN"), (2048, 2048, 2048, "NN"),
    (8192, 1024, 8192, "NN"), (1024, 8192, 256, "NN"), (2944, 2944, 1000, "NN"),
    (4097, 4097, 4097, "NN"), (6000, 6000, 2000, "NN"),
)


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
