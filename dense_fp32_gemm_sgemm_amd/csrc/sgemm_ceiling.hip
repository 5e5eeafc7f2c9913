// sgemm_ceiling.hip -- microbenchmarks that measure the ceilings SGEMM is
// measured against on this GPU.
//
// The Tinyforge README (results table and the note below it) makes the point
// that a percentage of a datasheet peak can be wrong by tens of percent and
// that the honest denominator is a measured pure-FMA ceiling.  These kernels
// measure, on gfx950:
//   * the FP32 matrix-core rate: back-to-back v_mfma_f32_32x32x2f32 or
//     v_mfma_f32_16x16x4f32 on 8 independent accumulators per wave;
//   * the FP32 vector rate: 16 independent v_fma_f32 chains per lane;
//   * the HBM rate: a 16-byte-per-lane streaming copy, which is also the
//     "plain copy of known size" used to calibrate the HBM byte counters,
//     and a read-only stream with eight 16-byte loads in flight per lane,
//     the roof for kernels that mostly read (a GEMM with few rows or
//     columns streams one operand and writes little);
//   * the dispatch floor: an empty kernel, the least time any launch takes.
// Every launch fills every SIMD of every CU: `blocks` workgroups of 256
// threads (four waves); callers pass a multiple of the CU count.
#include "../../include/sgemm_ceiling.h"
#include "sgemm_common.hpp"

namespace sg950 {

constexpr int kCeilThreads = 256;
constexpr int kChains = 8;

__global__ __launch_bounds__(kCeilThreads) void mfma32_ceiling_kernel(float *sink, int iters) {
  const float a = 1.0e-3f * (float)(threadIdx.x & 7);
  const float b = 1.0e-3f * (float)((threadIdx.x >> 3) & 7);
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kCeilThreads) void mfma16_ceiling_kernel(float *sink, int iters) {
  const float a = 1.0e-3f * (float)(threadIdx.x & 7);
  const float b = 1.0e-3f * (float)((threadIdx.x >> 3) & 7);
  floatx4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

constexpr int kFmaChains = 16;

__global__ __launch_bounds__(kCeilThreads) void fma_ceiling_kernel(float *sink, int iters) {
  float x[kFmaChains];
  const float m = 0.999f;
  const float d = 1.0e-3f * (float)(threadIdx.x & 15);
#pragma unroll
  for (int c = 0; c < kFmaChains; ++c) x[c] = (float)c;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kFmaChains; ++c) x[c] = fmaf(x[c], m, d);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kFmaChains; ++c) s += x[c];
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kCeilThreads) void copy_kernel(const floatx4 *__restrict__ src,
                                                            floatx4 *__restrict__ dst, long long n4) {
  const long long stride = (long long)gridDim.x * kCeilThreads;
  for (long long i = (long long)blockIdx.x * kCeilThreads + threadIdx.x; i < n4; i += stride)
    dst[i] = src[i];
}

// Read-only stream: each lane keeps kReadDepth 16-byte loads in flight per
// step and folds them into one sum (written per thread, so the loads stay
// live).  A grid-stride loop over whole steps; the rest (fewer than one
// step of the grid) is read one vector at a time.
constexpr int kReadDepth = 8;

__global__ __launch_bounds__(kCeilThreads) void read_kernel(const floatx4 *__restrict__ src, long long n4,
                                                            float *__restrict__ sink) {
  const long long nthreads = (long long)gridDim.x * kCeilThreads;
  const long long tid = (long long)blockIdx.x * kCeilThreads + threadIdx.x;
  const long long step = nthreads * kReadDepth;
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  long long base = 0;
  for (; base + step <= n4; base += step) {
    floatx4 v[kReadDepth];
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) v[u] = __builtin_nontemporal_load(src + base + u * nthreads + tid);
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) acc += v[u];
  }
  for (long long i = base + tid; i < n4; i += nthreads) acc += src[i];
  sink[tid] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Does nothing: its duration is the dispatch floor of a launch.
__global__ void empty_kernel() {}

}  // namespace sg950

extern "C" {

int sgemm_ceiling_mfma(int shape, int blocks, int iters, float *sink, void *stream,
                       double *flops_out) {
  if ((shape != 32 && shape != 16) || blocks <= 0 || iters <= 0) return SGEMM_CEIL_ERR_ARG;
  if (sink == nullptr) return SGEMM_CEIL_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double waves = (double)blocks * (sg950::kCeilThreads / 64);
  const double per_instr = (shape == 32) ? 32.0 * 32.0 * 2.0 * 2.0 : 16.0 * 16.0 * 4.0 * 2.0;
  if (flops_out) *flops_out = waves * (double)iters * sg950::kChains * per_instr;
  if (shape == 32)
    hipLaunchKernelGGL(sg950::mfma32_ceiling_kernel, dim3(blocks), dim3(sg950::kCeilThreads), 0, s, sink, iters);
  else
    hipLaunchKernelGGL(sg950::mfma16_ceiling_kernel, dim3(blocks), dim3(sg950::kCeilThreads), 0, s, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : SGEMM_CEIL_ERR_LAUNCH;
}

int sgemm_ceiling_fma(int blocks, int iters, float *sink, void *stream, double *flops_out) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return SGEMM_CEIL_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (flops_out)
    *flops_out = (double)blocks * sg950::kCeilThreads * (double)iters * sg950::kFmaChains * 2.0;
  hipLaunchKernelGGL(sg950::fma_ceiling_kernel, dim3(blocks), dim3(sg950::kCeilThreads), 0, s, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : SGEMM_CEIL_ERR_LAUNCH;
}

int sgemm_ceiling_copy(const float *src, float *dst, long long n, int blocks, void *stream) {
  if (src == nullptr || dst == nullptr || n < 0 || (n % 4) != 0 || blocks <= 0) return SGEMM_CEIL_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
    return SGEMM_CEIL_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sg950::copy_kernel, dim3(blocks), dim3(sg950::kCeilThreads), 0, s,
                     reinterpret_cast<const sg950::floatx4 *>(src),
                     reinterpret_cast<sg950::floatx4 *>(dst), n / 4);
  return hipGetLastError() == hipSuccess ? 0 : SGEMM_CEIL_ERR_LAUNCH;
}

int sgemm_ceiling_read(const float *src, long long n, int blocks, float *sink, void *stream) {
  if (src == nullptr || sink == nullptr || n < 0 || (n % 4) != 0 || blocks <= 0) return SGEMM_CEIL_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(src) & 15) return SGEMM_CEIL_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sg950::read_kernel, dim3(blocks), dim3(sg950::kCeilThreads), 0, s,
                     reinterpret_cast<const sg950::floatx4 *>(src), n / 4, sink);
  return hipGetLastError() == hipSuccess ? 0 : SGEMM_CEIL_ERR_LAUNCH;
}

int sgemm_ceiling_empty(int blocks, void *stream) {
  if (blocks <= 0) return SGEMM_CEIL_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sg950::empty_kernel, dim3(blocks), dim3(64), 0, s);
  return hipGetLastError() == hipSuccess ? 0 : SGEMM_CEIL_ERR_LAUNCH;
}

}  // extern "C"
