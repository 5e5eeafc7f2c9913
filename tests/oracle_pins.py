"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes a loaded oracle library and raises AssertionError when the
oracle disagrees with something the pages or the mathematics fix:

  * exact integer arithmetic (Python ints) by brute force over every 2x2x2
    problem with entries in {-1, 0, 1};
  * exact rational arithmetic (``fractions.Fraction``) on random tiny shapes
    with real fp32 values, within the oracle's own fp64 rounding bound;
  * closed forms (all-ones, arithmetic-series columns);
  * structure: identity, permutation and rank-1 operands;
  * a float64 library matmul (numpy) on a 512^3 problem;
  * the BLAS-style readings of the silent cases (alpha = 0, beta = 0, K = 0,
    leading-dimension gaps never read);
  * invariants of the denominator and of transposition.

The set is chosen so that each plausible single mistake (a dropped term, a
wrong sign or index, a transposed operand, a wrong leading dimension, the
scalars applied to the wrong term) fails at least one pin:
``tests/test_oracle.py`` builds such planted-mistake variants of the C file and
checks exactly that.  Run as a script (``python tests/oracle_pins.py LIB``) it
loads LIB, runs every pin and exits with the number of failed pins.
"""
from __future__ import annotations

import itertools
import os
import sys
from fractions import Fraction

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
from workloads import draw, padded  # noqa: E402

U53 = 2.0 ** -53


def _exact_product(A, B, C, alpha, beta):
    """Exact rationals: (alpha*A@B + beta*C, sum_k |A_ik B_kj|, |beta C_ij|)
    as nested lists (C may be None)."""
    M, K = A.shape
    N = B.shape[1]
    fa, fb = Fraction(float(alpha)), Fraction(float(beta))
    out, sab, sbc = [], [], []
    for i in range(M):
        row, arow, brow = [], [], []
        for j in range(N):
            s = Fraction(0)
            d = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                s += p
                d += abs(p)
            bc = fb * Fraction(float(C[i, j])) if (C is not None and beta != 0) else Fraction(0)
            row.append(fa * s + bc)
            arow.append(d)
            brow.append(abs(bc))
        out.append(row)
        sab.append(arow)
        sbc.append(brow)
    return out, sab, sbc


def pin_bruteforce_2x2x2(lib):
    """All 3^8 problems with A, B in {-1,0,1}^(2x2), against Python ints;
    each also with an integer C and alpha=2, beta=-3."""
    vals = (-1.0, 0.0, 1.0)
    rng = np.random.default_rng(7)
    for entries in itertools.product(vals, repeat=8):
        A = np.array(entries[:4], np.float32).reshape(2, 2)
        B = np.array(entries[4:], np.float32).reshape(2, 2)
        ai = [[int(x) for x in r] for r in A]
        bi = [[int(x) for x in r] for r in B]
        want = [[ai[i][0] * bi[0][j] + ai[i][1] * bi[1][j] for j in range(2)] for i in range(2)]
        ref, den = oracle.gemm(A, B, lib=lib)
        assert ref.tolist() == want, (entries, ref, want)
        wden = [[abs(ai[i][0] * bi[0][j]) + abs(ai[i][1] * bi[1][j]) for j in range(2)]
                for i in range(2)]
        assert den.tolist() == wden, (entries, den, wden)
        C = rng.integers(-1, 2, (2, 2)).astype(np.float32)
        ref2, den2 = oracle.gemm(A, B, C, 2.0, -3.0, lib=lib)
        want2 = [[2 * want[i][j] - 3 * int(C[i, j]) for j in range(2)] for i in range(2)]
        assert ref2.tolist() == want2, (entries, ref2, want2)
        wden2 = [[wden[i][j] + 3 * abs(int(C[i, j])) for j in range(2)] for i in range(2)]
        assert den2.tolist() == wden2, (entries, den2, wden2)


def pin_tiny_fractions(lib):
    """Random (M,N,K) in 1..6 with fp32 values, against exact rationals."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        M, N, K = (int(x) for x in rng.integers(1, 7, 3))
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        C = rng.standard_normal((M, N)).astype(np.float32)
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = float(np.float32(rng.uniform(-2, 2))) if trial % 3 else 0.0
        ref, den = oracle.gemm(A, B, C, alpha, beta, lib=lib)
        exact, sab, sbc = _exact_product(A, B, C, alpha, beta)
        for i in range(M):
            for j in range(N):
                scale = abs(alpha) * float(sab[i][j]) + float(sbc[i][j])
                bound = (K + 3) * 2 * U53 * scale + 1e-300
                err = abs(Fraction(float(ref[i, j])) - exact[i][j])
                assert float(err) <= bound, (trial, M, N, K, i, j, float(err), bound)
                eden = sab[i][j] + sbc[i][j]
                derr = abs(Fraction(float(den[i, j])) - eden)
                assert float(derr) <= (K + 2) * 2 * U53 * float(eden) + 1e-300


def pin_closed_forms(lib):
    """ones @ ones = K; ones @ (B[k,j] = k) = K(K-1)/2; both exact."""
    for M, N, K in ((3, 5, 1000), (1, 1, 1), (7, 2, 4097)):
        A = np.ones((M, K), np.float32)
        B = np.ones((K, N), np.float32)
        ref, den = oracle.gemm(A, B, lib=lib)
        assert np.all(ref == K) and np.all(den == K)
        Bk = np.repeat(np.arange(K, dtype=np.float32)[:, None], N, axis=1)
        ref, _ = oracle.gemm(A, Bk, lib=lib)
        assert np.all(ref == K * (K - 1) // 2), (ref.ravel()[:4], K * (K - 1) // 2)
        # alternating signs: sum_k (-1)^k = K mod 2
        As = np.tile(np.array([1.0, -1.0], np.float32), K // 2 + 1)[:K][None, :].repeat(M, 0)
        ref, den = oracle.gemm(np.ascontiguousarray(As), B, lib=lib)
        assert np.all(ref == K % 2) and np.all(den == K)


def pin_identity(lib):
    """A = I: C_ref = alpha*B + beta*C, exact on integer data."""
    rng = np.random.default_rng(3)
    n, N = 37, 23
    A = np.eye(n, dtype=np.float32)
    B = rng.integers(-9, 10, (n, N)).astype(np.float32)
    C = rng.integers(-9, 10, (n, N)).astype(np.float32)
    ref, _ = oracle.gemm(A, B, C, 3.0, -2.0, lib=lib)
    assert np.array_equal(ref, 3.0 * B.astype(np.int64) - 2.0 * C.astype(np.int64))
    Br = rng.uniform(-1, 1, (n, N)).astype(np.float32)
    ref, _ = oracle.gemm(A, Br, lib=lib)
    assert np.array_equal(ref, Br.astype(np.float64))
    # B = I on the right: C_ref = A exactly
    A2 = rng.uniform(-1, 1, (N, n)).astype(np.float32)
    ref, _ = oracle.gemm(A2, A, lib=lib)
    assert np.array_equal(ref, A2.astype(np.float64))


def pin_permutations(lib):
    """A = P permutes the rows of B; B = Q permutes the columns of A; exact."""
    rng = np.random.default_rng(5)
    M, K, N = 19, 19, 31
    perm = rng.permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1.0
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    ref, _ = oracle.gemm(P, B, lib=lib)
    assert np.array_equal(ref, B[perm].astype(np.float64))
    A = rng.uniform(-1, 1, (13, K)).astype(np.float32)
    q = rng.permutation(K)
    Q = np.zeros((K, K), np.float32)
    Q[q, np.arange(K)] = 1.0       # column j of Q picks row q[j]
    ref, _ = oracle.gemm(A, Q, lib=lib)
    assert np.array_equal(ref, A[:, q].astype(np.float64))


def pin_rank1(lib):
    """A = u v^T, B = w z^T: C_ref = alpha u_i z_j (v.w) + beta C, exact."""
    rng = np.random.default_rng(9)
    M, K, N = 11, 29, 17
    u = rng.integers(-3, 4, M)
    v = rng.integers(-3, 4, K)
    w = rng.integers(-3, 4, K)
    z = rng.integers(-3, 4, N)
    A = np.outer(u, v).astype(np.float32)
    B = np.outer(w, z).astype(np.float32)
    C = rng.integers(-5, 6, (M, N)).astype(np.float32)
    ref, _ = oracle.gemm(A, B, C, 2.0, 5.0, lib=lib)
    want = 2 * np.outer(u, z) * int(v @ w) + 5 * C.astype(np.int64)
    assert np.array_equal(ref, want.astype(np.float64))


def pin_numpy_float64(lib):
    """Against numpy's float64 matmul (a library routine), 512^3 and ragged."""
    for (M, N, K), seed in (((512, 512, 512), 1), ((127, 129, 17), 2), ((1, 300, 700), 3)):
        A, B, C = draw(M, N, K, seed=seed, with_c=True)
        ref, den = oracle.gemm(A, B, C, 1.5, 0.5, lib=lib)
        lib_ref = 1.5 * (A.astype(np.float64) @ B.astype(np.float64)) + 0.5 * C.astype(np.float64)
        assert np.max(np.abs(ref - lib_ref) / den) <= 1e-12
        lib_den = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)) + np.abs(0.5 * C)
        assert np.max(np.abs(den - lib_den) / lib_den) <= 1e-12


def pin_silent_cases(lib):
    """alpha = 0 / K = 0 do not read A, B; beta = 0 does not read C."""
    rng = np.random.default_rng(13)
    M, N, K = 6, 5, 4
    Anan = np.full((M, K), np.nan, np.float32)
    Bnan = np.full((K, N), np.nan, np.float32)
    C = rng.integers(-4, 5, (M, N)).astype(np.float32)
    ref, den = oracle.gemm(Anan, Bnan, C, 0.0, 0.5, lib=lib)
    assert np.array_equal(ref, 0.5 * C.astype(np.float64))
    assert np.array_equal(den, np.abs(0.5 * C.astype(np.float64)))
    ref, _ = oracle.gemm(Anan, Bnan, C, 0.0, 0.0, lib=lib)
    assert np.all(ref == 0.0)
    A0 = np.zeros((M, 0), np.float32)
    B0 = np.zeros((0, N), np.float32)
    ref, _ = oracle.gemm(A0, B0, C, 1.0, -2.0, lib=lib)
    assert np.array_equal(ref, -2.0 * C.astype(np.float64))
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    Cnan = np.full((M, N), np.nan, np.float32)
    ref, den = oracle.gemm(A, B, Cnan, 1.0, 0.0, lib=lib)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(den))
    ref_none, _ = oracle.gemm(A, B, None, 1.0, 0.0, lib=lib)
    assert np.array_equal(ref, ref_none)


def pin_leading_dims(lib):
    """NaN-poisoned gaps between the row length and the leading dimension are
    never read, and each matrix uses its own leading dimension."""
    rng = np.random.default_rng(17)
    M, N, K = 9, 7, 5
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    C = rng.integers(-4, 5, (M, N)).astype(np.float32)
    base, bden = oracle.gemm(A, B, C, 2.0, 3.0, lib=lib)
    for lda, ldb, ldc in ((K + 3, N, N), (K, N + 5, N), (K, N, N + 2), (K + 1, N + 9, N + 4),
                          (K + 7, N + 1, N + 11)):
        Ap, Bp, Cp = padded(A, lda), padded(B, ldb), padded(C, ldc)
        ref, den = oracle.gemm(Ap, Bp, Cp, 2.0, 3.0, lib=lib)
        assert np.array_equal(ref, base), (lda, ldb, ldc)
        assert np.array_equal(den, bden), (lda, ldb, ldc)


def pin_denominator_and_transpose(lib):
    """For non-negative data D = C_ref; D ignores signs; (AB)^T = B^T A^T."""
    rng = np.random.default_rng(19)
    M, N, K = 23, 17, 41
    A = rng.uniform(0, 1, (M, K)).astype(np.float32)
    B = rng.uniform(0, 1, (K, N)).astype(np.float32)
    C = rng.uniform(0, 1, (M, N)).astype(np.float32)
    ref, den = oracle.gemm(A, B, C, 1.0, 0.5, lib=lib)
    assert np.array_equal(ref, den)
    sA = np.where(rng.integers(0, 2, A.shape) == 1, A, -A).astype(np.float32)
    sC = -C
    ref2, den2 = oracle.gemm(sA, B, sC, 1.0, 0.5, lib=lib)
    assert np.array_equal(den2, den)
    assert not np.array_equal(ref2, ref)
    At = np.ascontiguousarray(A.T)
    Bt = np.ascontiguousarray(B.T)
    r1, _ = oracle.gemm(A, B, lib=lib)
    r2, _ = oracle.gemm(Bt, At, lib=lib)
    assert np.array_equal(r1, r2.T)


def pin_row_and_column_forms(lib):
    """The row- and column-selection forms agree with the full product."""
    A, B, C = draw(40, 33, 29, seed=23, with_c=True)
    full, fden = oracle.gemm(A, B, C, 1.5, 0.5, lib=lib)
    rows = [0, 39, 7, 7, 21]
    r, rd = oracle.gemm(A, B, C, 1.5, 0.5, rows=rows, lib=lib)
    assert np.array_equal(r, full[rows]) and np.array_equal(rd, fden[rows])
    cols = [32, 0, 5, 16]
    c, cd = oracle.gemm(A, B, C, 1.5, 0.5, cols=cols, lib=lib)
    assert np.array_equal(c, full[:, cols]) and np.array_equal(cd, fden[:, cols])


PINS = [pin_bruteforce_2x2x2, pin_tiny_fractions, pin_closed_forms, pin_identity,
        pin_permutations, pin_rank1, pin_numpy_float64, pin_silent_cases,
        pin_leading_dims, pin_denominator_and_transpose, pin_row_and_column_forms]


def run_all(lib):
    """Names of the pins that fail (an exception of any kind counts)."""
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception:  # noqa: BLE001 -- any failure means the pin caught it
            failed.append(pin.__name__)
    return failed


if __name__ == "__main__":
    path = sys.argv[1] if len(sys.argv) > 1 else None
    lib = oracle.load(path)
    bad = run_all(lib)
    print("failed pins:", ",".join(bad) if bad else "none")
    sys.exit(len(bad))
