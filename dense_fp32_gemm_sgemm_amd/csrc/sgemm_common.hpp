// sgemm_common.hpp -- types and small device helpers shared by the SGEMM kernels.
//
// Written for gfx950 (CDNA4): 64-lane wavefronts, 256 compute units in 8
// accelerator complex dies (XCDs) with a separate L2 each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sg950 {

// The GEMM problem C = alpha*op(A)*op(B) + beta*C, row-major, as one kernel
// argument.  op(A) is M x K: A itself (element (i,k) at A[i*lda + k]) when
// ta == 0, or the transpose of the K x M matrix A (element (i,k) at
// A[k*lda + i]) when ta == 1; likewise op(B) is K x N, from B (element (k,j)
// at B[k*ldb + j]) or, when tb == 1, from the N x K matrix B (element (k,j)
// at B[j*ldb + k]).
//
// Batches: `batch` independent problems of this shape, slice z using
// A + z*sa, B + z*sb and C + z*sc (element strides); kernels take the slice
// from blockIdx.z.  A single problem has batch = 1 and zero strides.
//
// Workspace: `ws` (ws_bytes bytes of device memory, or NULL) is scratch a
// call may use for the fixed-order split of its last round of tiles; only
// kernels that take that form read it.
struct Problem {
  int M, N, K;
  float alpha, beta;
  const float *A;
  int lda;
  const float *B;
  int ldb;
  float *C;
  int ldc;
  int ta, tb;
  long long sa, sb, sc;
  int batch;
  void *ws = nullptr;
  unsigned long long ws_bytes = 0;
};

// The fixed-order split of the last round of output tiles ("tail"): the
// first dp_tiles tiles run whole, one workgroup each; every other tile is
// split into `splits` K ranges, one workgroup each: with nkf = K / BK whole
// slabs, range s covers slabs [s*nkf/splits, (s+1)*nkf/splits) and the last
// range also the ragged rest of K.  Each of those writes its partial tile to
// `part`, then counts itself in flags[tile]; the one that counts last adds
// the partials in range order and writes the tile of C.
struct TailArgs {
  int dp_tiles = 0;
  int splits = 1;
  unsigned *flags = nullptr;
  float *part = nullptr;
};

// Moves the operand pointers to batch slice blockIdx.z.
__device__ __forceinline__ void select_slice(Problem &p) {
  const size_t z = blockIdx.z;
  p.A += z * (size_t)p.sa;
  p.B += z * (size_t)p.sb;
  p.C += z * (size_t)p.sc;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kNumXcds = 8;

// Workgroups are handed to the XCDs round-robin (workgroup w runs on XCD
// w % 8).  This remaps the hardware order so that XCD x receives a contiguous
// run of logical tile ids; with the grouped tile order below, the tiles that
// share one L2 then share rows of A and columns of B.
__device__ __forceinline__ int xcd_remap(int wg, int num_wg) {
  const int per_xcd = (num_wg + kNumXcds - 1) / kNumXcds;
  const int tall = num_wg - (per_xcd - 1) * kNumXcds;  // XCDs holding per_xcd ids
  const int xcd = wg % kNumXcds;
  const int local = wg / kNumXcds;
  return (xcd < tall) ? xcd * per_xcd + local
                      : tall * per_xcd + (xcd - tall) * (per_xcd - 1) + local;
}

// Grouped tile order: consecutive logical ids walk down `group_m` tile rows
// before moving one tile column right, so a window of consecutive ids covers a
// compact block of C.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int group_m,
                                             int &tm, int &tn) {
  const int per_group = group_m * tiles_n;
  const int g = id / per_group;
  const int first_m = g * group_m;
  const int rows = min(tiles_m - first_m, group_m);
  const int in_group = id - g * per_group;
  tm = first_m + in_group % rows;
  tn = in_group / rows;
}

// Launch planning (host side).  An entry point first runs every launcher of
// a call with `dry` set: each launch then only checks its grid against the
// HIP limits and records a failure, and nothing is enqueued.  Only when every
// launch of every batch chunk fits does it run the launchers again for real,
// so a call never leaves C partly updated behind a grid error.
struct LaunchPlan {
  bool dry = false;
  bool failed = false;
};
inline LaunchPlan &launch_plan() {
  static thread_local LaunchPlan plan;
  return plan;
}
// HIP grid limits: each dimension's work-items (blocks x threads) below 2^32,
// and at most 65535 blocks along y and z.
inline bool grid_fits(dim3 grid, dim3 block) {
  const unsigned long long lim = 0xffffffffULL;
  return grid.x >= 1 && grid.y >= 1 && grid.z >= 1 && grid.y <= 65535 && grid.z <= 65535 &&
         (unsigned long long)grid.x * block.x <= lim && (unsigned long long)grid.y * block.y <= lim &&
         (unsigned long long)grid.z * block.z <= lim;
}
// Every GEMM-path kernel launch goes through this macro.
#define SG950_LAUNCH(kernel, grid, block, shmem, stream, ...)                       \
  do {                                                                              \
    if (!::sg950::grid_fits((grid), (block))) {                                     \
      ::sg950::launch_plan().failed = true;                                         \
    } else if (!::sg950::launch_plan().dry) {                                       \
      hipLaunchKernelGGL(kernel, (grid), (block), (shmem), (stream), __VA_ARGS__); \
    }                                                                               \
  } while (0)

// Epilogue for one element: alpha*acc (+ beta*C when beta != 0; C is not read
// otherwise).
__device__ __forceinline__ void store_out(float *c, float acc, float alpha, float beta) {
  float v = alpha * acc;
  if (beta != 0.0f) v = fmaf(beta, *c, v);
  *c = v;
}

}  // namespace sg950
