/*
 * sgemm.h -- single-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined in "The road to a fast GEMM" (section "The
 * problem and the ceiling"):
 *
 *     C = alpha * A * B + beta * C
 *
 * with A of size MxK, B of size KxN and C of size MxN, every matrix row-major
 * FP32.  Each C[i,j] is the dot product of row i of A and column j of B
 * ("Optimizing SGEMM in CUDA", section "What is a SGEMM?").  The pages' kernels
 * take (M, N, K, alpha, A, B, beta, C) with packed rows; this interface adds a
 * leading dimension per matrix, as the vendor call on those pages does
 * ("Optimizing SGEMM in CUDA", section "cuBLAS implementation"), and a stream.
 *
 * Layout.  Element (i,k) of A is A[i*lda + k], element (k,j) of B is
 * B[k*ldb + j], element (i,j) of C is C[i*ldc + j].  Elements in the gap between
 * a row's length and its leading dimension are never read or written.
 *
 * Ownership.  Every matrix pointer is a device pointer on the calling thread's
 * current HIP device, owned by the caller.  The library allocates no device
 * memory, keeps no per-call state (its one setting is the process-wide
 * atomics mode below) and may be called from several threads.
 *
 * Asynchrony.  A call validates its arguments on the host, enqueues its
 * kernel(s) on `stream` (a hipStream_t; NULL means the default stream) and
 * returns without synchronising.  C must not overlap A or B.  Everything a
 * call enqueues is a kernel launch (C is cleared or scaled by a kernel, never
 * by a memset or copy), so calls may be captured into a HIP graph once one
 * ordinary call on the device has checked it.
 *
 * Arithmetic.  Strict FP32: products and sums are IEEE single precision with
 * round-to-nearest-even (fused multiply-add where the hardware fuses); no input
 * is rounded to a narrower format.  The order of the K-sum is unspecified, so
 * results on real-valued data may differ from another correct implementation
 * by rounding; on integer-valued data whose partial sums stay below 2^24 they
 * are exact.  Repeating a call gives bitwise the same C, except on the
 * variants that split K over workgroups (names ending in "_splitk", and the
 * split form of the few-rows kernel for M <= 8 with a large B, chosen
 * automatically when there are few output tiles and a long K): their partial
 * sums are added into C with atomics in the order the hardware runs them.
 * sgemm_set_atomics_mode(SGEMM_ATOMICS_NOT_ALLOWED) keeps the automatic
 * choice off those forms, so that every repeated call is bitwise the same.
 *
 * Special cases (BLAS conventions; the pages are silent on them):
 *   - M == 0 or N == 0: nothing is done.
 *   - alpha == 0 or K == 0: A and B are not read; C = beta * C.
 *   - beta == 0: C is not read, so NaN or Inf already in C does not propagate.
 *   - beta == 1 with alpha == 0 or K == 0: nothing is enqueued.
 *
 * Errors.  Every function returns SGEMM_OK (0) or a negative status; nothing
 * aborts or prints.  Argument errors are detected before any HIP call, and
 * so are grids too large to launch (SGEMM_ERR_GRID): every launch a call
 * needs, for every chunk of a large batch, is checked against the HIP grid
 * limits before the first one is enqueued, so an error never leaves C partly
 * updated.  SGEMM_ERR_LAUNCH reports a launch the runtime rejected anyway.
 */
#ifndef SGEMM_GFX950_H
#define SGEMM_GFX950_H

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_OK 0
#define SGEMM_ERR_DIM (-1)     /* M, N, K or batch negative */
#define SGEMM_ERR_LD (-2)      /* a leading dimension shorter than the stored row */
#define SGEMM_ERR_PTR (-3)     /* a matrix that must be read or written is NULL */
#define SGEMM_ERR_LAUNCH (-4)  /* the HIP runtime rejected a kernel launch */
#define SGEMM_ERR_DEVICE (-5)  /* the current device is not gfx950, or no device */
#define SGEMM_ERR_VARIANT (-6) /* sgemm_ex: variant index out of range */
#define SGEMM_ERR_OP (-7)      /* sgemm_op: opA or opB not SGEMM_OP_N / SGEMM_OP_T */
#define SGEMM_ERR_STRIDE (-8)  /* batched: a negative stride, or slices of C overlap */
#define SGEMM_ERR_GRID (-9)    /* the problem needs a launch grid beyond the HIP limits;
                                  nothing was enqueued */
#define SGEMM_ERR_WORKSPACE (-10) /* a workspace that is not 16-byte aligned, or (no-alloc
                                     entry point) a call needing more than the static scratch */

/* Operand orientation for sgemm_op: use the matrix as stored, or its transpose. */
#define SGEMM_OP_N 0
#define SGEMM_OP_T 1

/*
 * C = alpha * A * B + beta * C on `stream`, with the kernel variant and tile
 * configuration chosen from the shape, the operands' alignment and beta.
 *
 *   M, N, K   matrix sizes (>= 0)
 *   alpha     scale of A*B
 *   A, lda    MxK matrix, row stride lda >= max(1, K) elements
 *   B, ldb    KxN matrix, row stride ldb >= max(1, N) elements
 *   beta      scale of the incoming C
 *   C, ldc    MxN matrix, read (when beta != 0) and written, ldc >= max(1, N)
 *   stream    hipStream_t to enqueue on; NULL = default stream
 *
 * Returns SGEMM_OK or a negative SGEMM_ERR_* status.
 */
int sgemm(int M, int N, int K, float alpha, const float *A, int lda,
          const float *B, int ldb, float beta, float *C, int ldc, void *stream);

/*
 * As sgemm(), but runs kernel variant `variant` (0 <= variant <
 * sgemm_num_variants()); -1 means the automatic choice.  Every variant accepts
 * every valid problem (any shape, leading dimension, alignment and operand
 * orientation), so the variants can be compared on the same inputs.
 */
int sgemm_ex(int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc,
             void *stream, int variant);

/*
 * C = alpha * op(A) * op(B) + beta * C with op(X) = X (SGEMM_OP_N) or its
 * transpose (SGEMM_OP_T); op(A) is M x K and op(B) is K x N.  The pages count
 * transposed operands among what a general SGEMM library covers (Tinyforge
 * README, the comparison with the vendor library) and use the transposition
 * identity to call a column-major library from row-major code ("Optimizing
 * SGEMM in CUDA", "cuBLAS implementation"; "The road to a fast GEMM", the
 * vendor call in "The complete code").
 *
 *   opA == SGEMM_OP_N: A is M x K, element (i,k) at A[i*lda + k], lda >= max(1,K)
 *   opA == SGEMM_OP_T: A is K x M, op(A)(i,k) = A[k*lda + i],     lda >= max(1,M)
 *   opB == SGEMM_OP_N: B is K x N, element (k,j) at B[k*ldb + j], ldb >= max(1,N)
 *   opB == SGEMM_OP_T: B is N x K, op(B)(k,j) = B[j*ldb + k],     ldb >= max(1,K)
 *   C is M x N as in sgemm(); everything else (ownership, asynchrony, special
 *   cases, errors) is as for sgemm().  sgemm() is sgemm_op(N, N, ...).
 *
 * A column-major caller computing C = A*B (all column-major) calls
 * sgemm_op(N, N, N_, M_, K_, alpha, B, ldb, A, lda, beta, C, ldc, stream):
 * a column-major matrix is the row-major storage of its transpose, and
 * (A*B)^T = B^T * A^T.
 */
int sgemm_op(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, void *stream);

/* As sgemm_op() with an explicit kernel variant (-1 = automatic). */
int sgemm_op_ex(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, void *stream,
                int variant);

/*
 * A batch of independent GEMMs of one shape (strided batched SGEMM, the
 * "batching" the Tinyforge README lists among what a general library covers):
 * for z in [0, batch),
 *
 *     C_z = alpha * op(A_z) * op(B_z) + beta * C_z
 *
 * with A_z = A + z*strideA, B_z = B + z*strideB, C_z = C + z*strideC (element
 * strides, >= 0; a stride of 0 shares one matrix among all slices).  Each slice
 * is laid out as in sgemm_op().  The slices of C must not overlap: with
 * batch > 1, strideC >= (M-1)*ldc + N, else SGEMM_ERR_STRIDE.  batch == 0 is a
 * no-op; everything else is as for sgemm_op().  All slices are computed by one
 * set of launches (the kernels take the slice from the grid), so small
 * matrices in large batches fill the GPU.
 */
int sgemm_strided_batched(int opA, int opB, int M, int N, int K, float alpha,
                          const float *A, int lda, long long strideA, const float *B, int ldb,
                          long long strideB, float beta, float *C, int ldc, long long strideC,
                          int batch, void *stream);

/* As sgemm_strided_batched() with an explicit kernel variant (-1 = automatic). */
int sgemm_strided_batched_ex(int opA, int opB, int M, int N, int K, float alpha,
                             const float *A, int lda, long long strideA, const float *B,
                             int ldb, long long strideB, float beta, float *C, int ldc,
                             long long strideC, int batch, void *stream, int variant);

/*
 * Strided batched SGEMM with a caller workspace.  Everything is as for
 * sgemm_strided_batched(), except that the call may use `workspace`
 * (workspace_bytes bytes of device memory on the current device, 16-byte
 * aligned, or NULL for none) to split the last, partial round of output
 * tiles over K.  A grid whose tiles fill the CUs' workgroup slots a whole
 * number of times and a bit more leaves most CUs idle in its last round
 * ((4095, 4097, 1023): 1056 tiles of 128x128 for 512 slots); with a
 * workspace the tiles of that round are split into K ranges that fill the
 * slots, the partial tiles go to the workspace, and the workgroup that
 * finishes a tile's ranges last adds them in range order and writes the
 * tile of C.  The pages name splitting K as the way to fill the GPU when the
 * output tiles cannot ("The road to a fast GEMM", "Where to go next").
 * Problems with few rows (matrix-vector-like, bound by streaming B) use the
 * workspace the same way.  At most 8 rows of an untransposed B: the
 * 32-column strips of the full-K kernel split into up to four K ranges when
 * the strips alone leave CUs idle (up to four rows), or, where K is long for
 * the columns or the columns very many, (256-column strip, K chunk)
 * workgroups.  Up to 32 rows and 8192 columns: the strips of the
 * matrix-core few-rows kernel (16 columns, or 32 or 64 past 2048 columns,
 * at most 128 of them) split into two to four K chunks, as many as keep one
 * workgroup per CU.  Either way the partials are added in range order by
 * the last range.
 *
 * Results are bitwise repeatable (each output is one sum in a fixed order; no
 * atomics touch C), in either atomics mode.  The automatic choice takes the
 * split form only for a single matrix (batch == 1), when the predicted rate
 * is higher and the workspace holds its partial tiles; otherwise the call
 * runs as without a workspace.
 *
 * The workspace must be zero-filled before its first use (e.g. allocated
 * with hipMalloc and cleared with hipMemset once); each call that uses it
 * leaves it ready for the next (the counters it holds are back at zero when
 * the call's kernels finish).  The caller owns it; calls that use one
 * workspace must not overlap in time (same stream, or synchronised).
 * A workspace that is not 16-byte aligned gives SGEMM_ERR_WORKSPACE; one that
 * is too small is not an error (the split form is not taken).
 */
int sgemm_strided_batched_ws(int opA, int opB, int M, int N, int K, float alpha,
                             const float *A, int lda, long long strideA, const float *B, int ldb,
                             long long strideB, float beta, float *C, int ldc, long long strideC,
                             int batch, void *workspace, unsigned long long workspace_bytes,
                             void *stream);

/* As sgemm_strided_batched_ws() with an explicit kernel variant (-1 = automatic). */
int sgemm_strided_batched_ws_ex(int opA, int opB, int M, int N, int K, float alpha,
                                const float *A, int lda, long long strideA, const float *B,
                                int ldb, long long strideB, float beta, float *C, int ldc,
                                long long strideC, int batch, void *workspace,
                                unsigned long long workspace_bytes, void *stream, int variant);

/* The variant sgemm_strided_batched_ws() would run with a workspace of
 * workspace_bytes bytes (no launch, no HIP call; see sgemm_select_variant). */
int sgemm_strided_batched_ws_select_variant(int opA, int opB, int M, int N, int K, float alpha,
                                            const float *A, int lda, long long strideA,
                                            const float *B, int ldb, long long strideB,
                                            float beta, const float *C, int ldc,
                                            long long strideC, int batch,
                                            unsigned long long workspace_bytes);

/*
 * sgemm_strided_batched_ws() for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is the library's own static scratch, 4 KiB +
 * 32 MiB per GPU, held from module load until the process ends.  The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating routine).
 *
 * Everything else is as for sgemm_strided_batched_ws() with that workspace:
 * the same automatic choice, results bitwise equal to it.  The split plans
 * are capped to fit the scratch, so no problem size needs more; a call that
 * would is refused with SGEMM_ERR_WORKSPACE before anything is enqueued.
 *
 * The first call on a device looks up the device's scratch address and
 * clears its counters with a small kernel on `stream` (one-time set-up);
 * every call leaves the counters at zero.  All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (on different streams, or
 * from several threads without ordering) race and give wrong results.
 */
int sgemm_strided_batched_noalloc(int opA, int opB, int M, int N, int K, float alpha,
                                  const float *A, int lda, long long strideA, const float *B,
                                  int ldb, long long strideB, float beta, float *C, int ldc,
                                  long long strideC, int batch, void *stream);

/*
 * Bytes of workspace the automatic choice of sgemm_strided_batched_ws() can
 * use for this problem (packed leading dimensions): 0 when it would not take
 * the split form, at most 4 KiB + 32 MiB for any problem, or a negative
 * SGEMM_ERR_* status for invalid operations or sizes.
 */
long long sgemm_workspace_size(int opA, int opB, int M, int N, int K, int batch);

/* Number of kernel variants, and a stable name for each ("" when out of range).
 * The variants are the kernel versions sgemm_ex() can force, as the pages'
 * benchmark walks its table of kernel versions ("The road to a fast GEMM",
 * "The complete code"). */
int sgemm_num_variants(void);
const char *sgemm_variant_name(int variant);

/*
 * The variant sgemm() would run for this problem (no launch, no HIP call), or
 * a negative SGEMM_ERR_* status for invalid arguments or a problem too large
 * to launch.  Returns -100 when the problem needs no GEMM kernel (M or N
 * zero, or alpha == 0 or K == 0).  Takes every argument sgemm() takes except
 * the stream: alpha because alpha == 0 needs no GEMM kernel, the pointers
 * because their alignment selects the load paths.  The pointers are not
 * dereferenced.  Its variant index names the registry of sgemm_variant_name,
 * the per-shape kernel table of the build (the pages keep such a registry
 * of their kernel versions, "The road to a fast GEMM", "The complete code").
 */
int sgemm_select_variant(int M, int N, int K, float alpha, const float *A,
                         int lda, const float *B, int ldb, float beta,
                         const float *C, int ldc);

/* sgemm_select_variant for sgemm_op problems. */
int sgemm_op_select_variant(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                            int lda, const float *B, int ldb, float beta, const float *C,
                            int ldc);

/* sgemm_select_variant for sgemm_strided_batched problems. */
int sgemm_strided_batched_select_variant(int opA, int opB, int M, int N, int K, float alpha,
                                         const float *A, int lda, long long strideA,
                                         const float *B, int ldb, long long strideB, float beta,
                                         const float *C, int ldc, long long strideC, int batch);

/* Short English description of a status code (never NULL).  The pages check
 * every runtime call with a macro that reports the error text ("The road to
 * a fast GEMM", "The complete code"); this is that text for the library's own
 * status codes. */
const char *sgemm_status_string(int status);

/* Interface version, currently 5 (2 added sgemm_op, 3 the strided batches, 4
 * the atomics mode, 5 the workspace entry points and SGEMM_ERR_GRID). */
int sgemm_version(void);

/*
 * Atomics mode, process-wide (default SGEMM_ATOMICS_ALLOWED).  The operation
 * fixes C = alpha*A*B + beta*C but not the order of the K-sum ("The road to a
 * fast GEMM", section "The problem and the ceiling"), so variants that split
 * K over workgroups and add their partial sums into C with atomics are
 * correct, but their last bits depend on the order the hardware runs the
 * adds.  With SGEMM_ATOMICS_NOT_ALLOWED the automatic choice (variant -1 and
 * the *_select_variant functions) takes only variants that write every
 * element of C once from sums formed in a fixed order, at some cost in speed
 * on problems with few output tiles and a long K; variants requested by
 * index run as asked.  sgemm_set_atomics_mode returns SGEMM_OK, or
 * SGEMM_ERR_OP for any other mode value (the mode is then unchanged).  The
 * mode is read once per call; a change made while another thread is inside
 * a call applies from that thread's next call.
 */
#define SGEMM_ATOMICS_NOT_ALLOWED 0
#define SGEMM_ATOMICS_ALLOWED 1
int sgemm_set_atomics_mode(int mode);
int sgemm_get_atomics_mode(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_GFX950_H */
