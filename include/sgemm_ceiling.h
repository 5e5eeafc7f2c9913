/*
 * sgemm_ceiling.h -- measured-ceiling microbenchmarks for the SGEMM library.
 *
 * The Tinyforge README (results table and the paragraph under it) measures its
 * GEMM against a ceiling it measured with a pure-FMA kernel rather than the
 * datasheet figure, because the two differed by about 30%.  These entry points
 * run the same kind of measurement on an MI355X: a launch does a known amount
 * of work, and the caller times it (with events on the same stream) to get a
 * sustained rate.  They live in the same shared library as sgemm().
 *
 * All pointers are device pointers on the current device, owned by the caller.
 * Each call only enqueues; it returns 0, SGEMM_CEIL_ERR_ARG for bad arguments
 * (checked before any HIP call) or SGEMM_CEIL_ERR_LAUNCH.
 */
#ifndef SGEMM_CEILING_H
#define SGEMM_CEILING_H

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_CEIL_ERR_ARG (-1)
#define SGEMM_CEIL_ERR_LAUNCH (-2)

/*
 * FP32 matrix-core ceiling: `blocks` workgroups of four waves, each wave
 * issuing `iters` rounds of 8 independent v_mfma_f32_32x32x2f32 (shape 32) or
 * v_mfma_f32_16x16x4f32 (shape 16).  `sink` receives blocks*256 floats (one
 * per thread, to keep the work live).  *flops_out (if not NULL) is set to the
 * launch's floating-point operation count.
 */
int sgemm_ceiling_mfma(int shape, int blocks, int iters, float *sink, void *stream,
                       double *flops_out);

/*
 * FP32 vector ceiling: each thread runs 16 independent v_fma_f32 chains for
 * `iters` steps.  `sink` and *flops_out as above.
 */
int sgemm_ceiling_fma(int blocks, int iters, float *sink, void *stream, double *flops_out);

/*
 * HBM streaming copy of n floats (n a multiple of 4, both pointers 16-byte
 * aligned) with a grid of `blocks` workgroups of 256 threads: reads 4n bytes
 * and writes 4n bytes.
 */
int sgemm_ceiling_copy(const float *src, float *dst, long long n, int blocks, void *stream);

/*
 * HBM read ceiling: streams n floats (n a multiple of 4, src 16-byte aligned)
 * with `blocks` workgroups of 256 threads, eight 16-byte loads in flight per
 * lane, and writes one partial sum per thread to `sink` (blocks*256 floats).
 * Reads 4n bytes; a buffer well past the 256 MB last-level cache makes
 * repeated launches read HBM.  maxxfuu ("Placing The Naive Kernel On The
 * Roofline") places kernels under a bandwidth roof, and the Tinyforge README
 * measures its roof rather than quoting it.
 */
int sgemm_ceiling_read(const float *src, long long n, int blocks, float *sink, void *stream);

/*
 * Dispatch floor: `blocks` workgroups of one wave that do nothing.  Its
 * duration is the least time any kernel launch occupies the GPU, the floor
 * under the smallest GEMMs of the sweep (the Tinyforge README warns that
 * small-size timings mostly measure such overheads).
 */
int sgemm_ceiling_empty(int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_CEILING_H */
