// sgemm_skinny.hip -- SGEMM with few rows of C (M <= 8): a matrix-vector-like
// product bound by the bandwidth of streaming B.
//
// With M <= 8 a GEMM does 2*M FLOP per element of B it reads, below the
// MI355X ridge point (about 20 FLOP/byte): the whole of B has to stream from
// HBM once, and the kernel's job is to keep enough loads in flight on every
// CU.  The work is split over columns of B (256 per workgroup: 64 lanes x a
// 16-byte vector, so each wavefront load is 1 KiB of one row) and over K
// (each workgroup takes a chunk of rows, its four waves a quarter of the chunk
// each).  A lane keeps M x 4 partial sums; the four waves' sums are added
// through LDS in a fixed order, and the workgroup adds alpha * sum into C with
// one float atomic per element.  C is first scaled by beta in a separate
// launch, so the result is beta*C + alpha*A*B with the K-chunks' partial sums
// added in an unspecified order (exact on integer data; within fp32 rounding
// otherwise).  A's values are the same for every lane and are read through
// the scalar path.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"

#include <climits>

namespace sg950 {

constexpr int kSkinnyCols = 256;  // columns of B per workgroup
constexpr int kSkinnyWaves = 4;

// TB: B is stored N x K (op(B) = its transpose); its elements are then read
// one by one along the column (correct, not bandwidth-efficient: the table
// never picks this kernel for a transposed B).
template <int MR, bool VB, bool TB>
__global__ __launch_bounds__(kSkinnyWaves * 64) void skinny_kernel(Problem p, int kchunk) {
  select_slice(p);
  __shared__ float red[kSkinnyWaves][MR][kSkinnyCols];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = blockIdx.x * kSkinnyCols + 4 * lane;
  const int kb = blockIdx.y * kchunk;
  const int ke = min(p.K, kb + kchunk);
  const int quarter = (kchunk + kSkinnyWaves - 1) / kSkinnyWaves;
  const int k0 = min(ke, kb + w * quarter);
  const int k1 = min(ke, k0 + quarter);

  // Columns past N read the last column (in bounds, never stored).
  int cc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cc[e] = min(c0 + e, p.N - 1);
  const bool vec = VB && !TB && (c0 + 3 < p.N);
  const size_t ldb = (size_t)p.ldb;
  const size_t sa_r = p.ta ? 1 : (size_t)p.lda, sa_k = p.ta ? (size_t)p.lda : 1;

  float acc[MR][4];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;

#pragma unroll 4
  for (int k = k0; k < k1; ++k) {
    floatx4 b;
    if (TB) {
      b = floatx4{p.B[(size_t)cc[0] * ldb + k], p.B[(size_t)cc[1] * ldb + k],
                  p.B[(size_t)cc[2] * ldb + k], p.B[(size_t)cc[3] * ldb + k]};
    } else {
      const float *brow = p.B + (size_t)k * ldb;
      if (vec) {
        b = *reinterpret_cast<const floatx4 *>(brow + c0);
      } else {
        b = floatx4{brow[cc[0]], brow[cc[1]], brow[cc[2]], brow[cc[3]]};
      }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (r < p.M) {
        const float a = p.A[(size_t)r * sa_r + (size_t)k * sa_k];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(a, b[e], acc[r][e]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][r][4 * lane + e] = acc[r][e];
  __syncthreads();
  if (w != 0) return;  // no barrier after this point
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (r >= p.M) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = red[0][r][4 * lane + e];
#pragma unroll
      for (int q = 1; q < kSkinnyWaves; ++q) s += red[q][r][4 * lane + e];
      if (c0 + e < p.N) atomicAdd(p.C + (size_t)r * (size_t)p.ldc + c0 + e, p.alpha * s);
    }
  }
}

// K rows per workgroup: enough workgroups (over all batch slices) for about
// four per CU, at least 64 rows (16 per wave) each, a multiple of 16.
static int skinny_kchunk(const Problem &p, long long strips) {
  const long long target = 1024;
  long long chunks = target / (strips * p.batch > 0 ? strips * p.batch : 1);
  if (chunks < 1) chunks = 1;
  long long kc = ((long long)p.K + chunks - 1) / chunks;
  if (kc < 64) kc = 64;
  kc = (kc + 15) / 16 * 16;
  return (int)kc;
}

int launch_skinny(const Problem &p, hipStream_t stream) {
  if (p.M > 8) return -1;
  const long long strips = ((long long)p.N + kSkinnyCols - 1) / kSkinnyCols;
  const int kc = skinny_kchunk(p, strips);
  const long long chunks = ((long long)p.K + kc - 1) / kc;
  if (strips > INT_MAX || chunks > 65535) return -1;
  // C = beta*C first (zeros when beta == 0, nothing when beta == 1).
  if (p.beta != 1.0f && launch_scale(p, stream) != 0) return -1;
  const dim3 grid((unsigned)strips, (unsigned)chunks, (unsigned)p.batch);
  const dim3 block(kSkinnyWaves * 64);
  const bool vb = b_vec_ok(p);
#define SG950_SKINNY(MR_)                                                                     \
  do {                                                                                        \
    if (p.tb)                                                                                 \
      hipLaunchKernelGGL((skinny_kernel<MR_, false, true>), grid, block, 0, stream, p, kc); \
    else if (vb)                                                                              \
      hipLaunchKernelGGL((skinny_kernel<MR_, true, false>), grid, block, 0, stream, p, kc); \
    else                                                                                      \
      hipLaunchKernelGGL((skinny_kernel<MR_, false, false>), grid, block, 0, stream, p, kc); \
  } while (0)
  if (p.M <= 1) {
    SG950_SKINNY(1);
  } else if (p.M <= 2) {
    SG950_SKINNY(2);
  } else if (p.M <= 4) {
    SG950_SKINNY(4);
  } else {
    SG950_SKINNY(8);
  }
#undef SG950_SKINNY
  return 0;
}

}  // namespace sg950
