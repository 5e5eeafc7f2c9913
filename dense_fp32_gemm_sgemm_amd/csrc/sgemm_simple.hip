// sgemm_simple.hip -- one output element per lane, and the C = beta*C kernel.
//
// The one-thread-per-output kernel is the starting point of every page ("The
// road to a fast GEMM", sections "v0 to v1: the naive version and
// coalescing"; "Optimizing SGEMM in CUDA", "Kernel 1"): a thread walks a row
// of A and a column of B.  What decides its speed is which matrix index runs
// along the lanes of a wavefront: here the 64 lanes of a wave take 64
// consecutive columns of one row of C, so each load of B and each store of C
// is one contiguous 256-byte access, and the load of A is a single address
// broadcast to all lanes.  It handles any shape, leading dimension and
// alignment (and either operand transposed, with strided reads) and serves
// the tiny problems where a tiled kernel would leave most of its tile empty.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"

namespace sg950 {

constexpr int kSimpleCols = 64;  // one wave along N
constexpr int kSimpleRows = 4;   // four waves per workgroup, one row each

__global__ __launch_bounds__(kSimpleCols *kSimpleRows) void simple_kernel(Problem p) {
  select_slice(p);
  // Element strides of op(A) along its rows / along K, and of op(B) along K /
  // along its columns (transposed operands swap them).
  const size_t sa_i = p.ta ? 1 : (size_t)p.lda, sa_k = p.ta ? (size_t)p.lda : 1;
  const size_t sb_k = p.tb ? 1 : (size_t)p.ldb, sb_j = p.tb ? (size_t)p.ldb : 1;
  // Grid-stride over row groups (x) and column blocks (y): the grid is capped
  // at the launch limits, so any M and N run.  No barrier in this kernel.
  for (long long rb = blockIdx.x; rb * kSimpleRows < p.M; rb += gridDim.x) {
    const int row = (int)(rb * kSimpleRows) + (threadIdx.x >> 6);
    if (row >= p.M) continue;
    for (long long cb = blockIdx.y; cb * kSimpleCols < p.N; cb += gridDim.y) {
      const int col = (int)(cb * kSimpleCols) + (threadIdx.x & (kSimpleCols - 1));
      if (col >= p.N) continue;
      const float *a = p.A + (size_t)row * sa_i;
      const float *b = p.B + (size_t)col * sb_j;
      float acc = 0.0f;
      int k = 0;
      // Four independent partial sums hide the FMA latency; they are combined
      // in a fixed order, so the result is still a plain fp32 sum of the K
      // products.
      float acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
      for (; k + 4 <= p.K; k += 4) {
        acc = fmaf(a[(size_t)k * sa_k], b[(size_t)k * sb_k], acc);
        acc1 = fmaf(a[(size_t)(k + 1) * sa_k], b[(size_t)(k + 1) * sb_k], acc1);
        acc2 = fmaf(a[(size_t)(k + 2) * sa_k], b[(size_t)(k + 2) * sb_k], acc2);
        acc3 = fmaf(a[(size_t)(k + 3) * sa_k], b[(size_t)(k + 3) * sb_k], acc3);
      }
      for (; k < p.K; ++k) acc = fmaf(a[(size_t)k * sa_k], b[(size_t)k * sb_k], acc);
      acc = (acc + acc1) + (acc2 + acc3);
      store_out(p.C + (size_t)row * p.ldc + col, acc, p.alpha, p.beta);
    }
  }
}

// C = beta * C (beta == 0 writes zeros without reading C), batch slice
// blockIdx.z at C + z*sc; grid-stride over rows and 64-column blocks.
__global__ __launch_bounds__(256) void scale_kernel(int M, int N, float beta, float *C, int ldc,
                                                   long long sc) {
  float *cz = C + (size_t)blockIdx.z * (size_t)sc;
  for (long long rb = blockIdx.x; rb * 4 < M; rb += gridDim.x) {
    const long long row = rb * 4 + (threadIdx.x >> 6);
    if (row >= M) continue;
    for (long long cb = blockIdx.y; cb * 64 < N; cb += gridDim.y) {
      const long long col = cb * 64 + (threadIdx.x & 63);
      if (col >= N) continue;
      float *c = cz + (size_t)row * (size_t)ldc + (size_t)col;
      *c = (beta == 0.0f) ? 0.0f : beta * *c;
    }
  }
}

// Grid extents of the two kernels above: enough blocks to cover the matrix,
// capped (the kernels stride over the rest).
constexpr long long kMaxStrideGridX = 1LL << 20, kMaxStrideGridY = 65535;

int launch_simple(const Problem &p, hipStream_t stream) {
  const long long gx = ((long long)p.M + kSimpleRows - 1) / kSimpleRows;
  const long long gy = ((long long)p.N + kSimpleCols - 1) / kSimpleCols;
  const dim3 grid((unsigned)(gx < kMaxStrideGridX ? gx : kMaxStrideGridX),
                  (unsigned)(gy < kMaxStrideGridY ? gy : kMaxStrideGridY), (unsigned)p.batch);
  SG950_LAUNCH(simple_kernel, grid, dim3(kSimpleCols * kSimpleRows), 0, stream, p);
  return 0;
}

int launch_scale(const Problem &p, hipStream_t stream) {
  const long long gx = ((long long)p.M + 3) / 4;
  const long long gy = ((long long)p.N + 63) / 64;
  const dim3 grid((unsigned)(gx < kMaxStrideGridX ? gx : kMaxStrideGridX),
                  (unsigned)(gy < kMaxStrideGridY ? gy : kMaxStrideGridY), (unsigned)p.batch);
  SG950_LAUNCH(scale_kernel, grid, dim3(256), 0, stream, p.M, p.N, p.beta, p.C, p.ldc, p.sc);
  return 0;
}

}  // namespace sg950
