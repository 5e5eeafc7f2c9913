/*
 * sgemm_oracle.c -- plain CPU reference for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test-suite, the smoke check and the CPU-baseline leg of the benchmark
 * load the library built from it.  It shares no source, header or helper with
 * the HIP library, and nothing here is ever called from the product path.
 *
 * What it computes.  "The road to a fast GEMM" (section "The problem and the
 * ceiling") defines the operation as C = alpha*A*B + beta*C with A of size MxK,
 * B of size KxN and C of size MxN, every matrix row-major FP32.  "Optimizing
 * SGEMM in CUDA" (section "What is a SGEMM?") says each C[i,j] is the dot
 * product of row i of A with column j of B.  Written out:
 *
 *     S[i,j]     = sum_{k=0}^{K-1} A[i,k] * B[k,j]
 *     C_ref[i,j] = alpha * S[i,j] + beta * C_in[i,j]
 *
 * Precision.  Every product of two floats is exact in double (24+24 <= 53
 * significand bits), so only the additions round; the result is within
 * K * 2^-53 * sum|A||B| of the exact value, far below the 1e-5 tolerance the
 * GPU result is held to.  The loop order is i, then k, then j with a per-row
 * double accumulator, the cache-friendly order the same page uses for its own
 * CPU reference (section "The complete code"); the i-loop is split across
 * OpenMP threads and nothing else is blocked, fused or reordered.
 *
 * Alongside C_ref it returns the per-element denominator of the tolerance,
 *     D[i,j] = sum_k |A[i,k]| * |B[k,j]| + |beta * C_in[i,j]| .
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - beta == 0: C_in is not read, the BLAS meaning of beta = 0, so a NaN in
 *     the output buffer does not leak into the result.
 *   - alpha == 0 or K == 0: A and B are not read; C_ref = beta * C_in.
 *   - leading dimensions: element (i,k) of A is A[i*lda + k], likewise for B
 *     and C; elements in the gaps between K (or N) and the leading dimension
 *     are never read.
 *
 * The test-suite also builds altered copies of this file, each with one
 * deliberate mistake patched into a temporary copy, to prove that the pins
 * catch such mistakes; this file itself holds only the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One output row i: s[j] = sum_k A[i,k] B[k,j], d[j] = sum_k |A[i,k] B[k,j]|,
 * both for j in [0, N). */
static void row_sums(int64_t i, int64_t N, int64_t K, const float *A,
                     int64_t lda, const float *B, int64_t ldb, double *s,
                     double *d) {
    memset(s, 0, (size_t)N * sizeof(double));
    memset(d, 0, (size_t)N * sizeof(double));
    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) {
            const double p = a * (double)brow[j];
            s[j] += p;
            d[j] += fabs(p);
        }
    }
}

/* Epilogue for one element: writes C_ref and D from the row sums. */
static void finish(double alpha, double beta, int use_ab, double s, double d,
                   const float *cin, double *cref, double *den) {
    double ab = use_ab ? alpha * s : 0.0;
    double bc = 0.0;
    if (beta != 0.0) bc = beta * (double)(*cin);
    *cref = ab + bc;
    *den = (use_ab ? d : 0.0) + fabs(bc);
}

/*
 * Rows form.  Computes C_ref and D for the output rows listed in rows[0..nrows)
 * (rows == NULL means every row 0..M-1, nrows is then ignored).  Output row r
 * (the r-th listed row) is written to cref[r*N .. r*N+N) and den[...] alike.
 * Cin may be NULL when beta == 0; A and B may be NULL when alpha == 0 or K == 0.
 * Returns 0, or -1 if a scratch allocation fails.
 */
int oracle_sgemm_rows(int64_t M, int64_t N, int64_t K, double alpha,
                      const float *A, int64_t lda, const float *B, int64_t ldb,
                      double beta, const float *Cin, int64_t ldc,
                      const int64_t *rows, int64_t nrows, double *cref,
                      double *den) {
    if (rows == NULL) nrows = M;
    if (nrows <= 0 || N <= 0) return 0;
    const int use_ab = (alpha != 0.0 && K > 0);
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *d = (double *)malloc((size_t)N * sizeof(double));
        if (s == NULL || d == NULL) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t i = rows ? rows[r] : r;
                if (use_ab) {
                    row_sums(i, N, K, A, lda, B, ldb, s, d);
                } else {
                    memset(s, 0, (size_t)N * sizeof(double));
                    memset(d, 0, (size_t)N * sizeof(double));
                }
                for (int64_t j = 0; j < N; ++j) {
                    const float *cin = Cin ? Cin + i * ldc + j : NULL;
                    finish(alpha, beta, use_ab, s[j], d[j], cin, cref + r * N + j,
                           den + r * N + j);
                }
            }
        }
        free(s);
        free(d);
    }
    return failed ? -1 : 0;
}

/*
 * Columns form.  Computes C_ref and D for every row and the output columns
 * listed in cols[0..ncols); element (i, c) goes to cref[i*ncols + c].  Used to
 * check sampled columns of products too large to compute whole.  Same
 * definition and precision as the rows form; the j-loop runs over the listed
 * columns only.
 */
int oracle_sgemm_cols(int64_t M, int64_t N, int64_t K, double alpha,
                      const float *A, int64_t lda, const float *B, int64_t ldb,
                      double beta, const float *Cin, int64_t ldc,
                      const int64_t *cols, int64_t ncols, double *cref,
                      double *den) {
    (void)N;
    if (M <= 0 || ncols <= 0) return 0;
    const int use_ab = (alpha != 0.0 && K > 0);
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double *s = (double *)malloc((size_t)ncols * sizeof(double));
        double *d = (double *)malloc((size_t)ncols * sizeof(double));
        if (s == NULL || d == NULL) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; ++i) {
                memset(s, 0, (size_t)ncols * sizeof(double));
                memset(d, 0, (size_t)ncols * sizeof(double));
                if (use_ab) {
                    for (int64_t k = 0; k < K; ++k) {
                        const double a = (double)A[i * lda + k];
                        const float *brow = B + k * ldb;
                        for (int64_t c = 0; c < ncols; ++c) {
                            const double p = a * (double)brow[cols[c]];
                            s[c] += p;
                            d[c] += fabs(p);
                        }
                    }
                }
                for (int64_t c = 0; c < ncols; ++c) {
                    const float *cin = Cin ? Cin + i * ldc + cols[c] : NULL;
                    finish(alpha, beta, use_ab, s[c], d[c], cin, cref + i * ncols + c,
                           den + i * ncols + c);
                }
            }
        }
        free(s);
        free(d);
    }
    return failed ? -1 : 0;
}
