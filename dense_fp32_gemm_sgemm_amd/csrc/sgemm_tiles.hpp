// sgemm_tiles.hpp -- global-memory loaders for one K-slab of an operand tile.
//
// A workgroup that owns a BM x BN tile of C walks K in slabs of BK: per slab
// it needs a BM x BK block of op(A) and a BK x BN block of op(B).  In memory
// each operand is row-major and comes in one of two orientations:
//   * "row" blocks: the block's rows run along M (or N) and K is contiguous
//     (A untransposed; B transposed, i.e. stored N x K);
//   * "k-row" blocks: the block's rows run along K and M (or N) is contiguous
//     (B untransposed; A transposed, i.e. stored K x M).
// Either way the threads read with lanes running along the contiguous
// dimension, four floats per lane, so a 64-lane wavefront issues one 16-byte
// load per lane covering whole 64- to 256-byte row segments ("The road to a
// fast GEMM", sections "v0 to v1" and "v5: vectorized loads", on letting the
// lane index run along the contiguous dimension and on 128-bit accesses).
//
// Edges.  Rows (or columns) past the matrix edge in M or N are clamped to the
// last valid one: those loads stay inside the matrix and only feed
// accumulators whose outputs are never stored.  K is different -- every k
// contributes to every output -- so in the last, partial slab the elements
// with k >= K are replaced by zero (selected, never multiplied, so a NaN or
// Inf in the matrix cannot leak in) and are not loaded at all.
//
// Alignment.  With V = true a lane loads its four floats as one 16-byte
// vector; that needs a 16-byte aligned base and a leading dimension that is a
// multiple of four (and, for k-row blocks, a row length that is one too, so a
// vector never crosses the end of a row).  With V = false the same four floats
// are loaded one by one, which works for any pointer and leading dimension.
#pragma once

#include "sgemm_common.hpp"

namespace sg950 {

// ROWS x BK block, element (r, k) at X[r*ld + k], NT threads; vector i of
// thread t covers block row (t + i*NT) / (BK/4), block columns
// 4*((t + i*NT) % (BK/4)) .. +3.
template <int ROWS, int BK, int NT, bool V>
struct RowTileLoader {
  static constexpr int kVecs = ROWS * BK / 4 / NT;
  static_assert((ROWS * BK / 4) % NT == 0, "tile must split evenly over the threads");
  static_assert(BK % 4 == 0, "BK must be a multiple of 4");

  const float *ptr[kVecs];  // element (row, 4-run start) at k = 0
  int kc[kVecs];            // k offset of the run inside the slab
  floatx4 v[kVecs];

  static __device__ __forceinline__ int row_of(int tid, int i) { return (tid + i * NT) / (BK / 4); }
  static __device__ __forceinline__ int col_of(int tid, int i) { return ((tid + i * NT) % (BK / 4)) * 4; }

  // X: the matrix, ld its leading dimension, nrows its number of rows (M or
  // N), r0 the block's first row.
  __device__ __forceinline__ void init(const float *X, int ld, int nrows, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int row = min(r0 + row_of(tid, i), nrows - 1);
      kc[i] = col_of(tid, i);
      ptr[i] = X + (size_t)row * (size_t)ld + kc[i];
    }
  }

  // Loads the slab starting at k0; TAIL marks the last slab when K % BK != 0.
  template <bool TAIL>
  __device__ __forceinline__ void load(int k0, int K) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const float *q = ptr[i] + k0;
      if (!TAIL) {
        if (V) {
          v[i] = *reinterpret_cast<const floatx4 *>(q);
        } else {
          v[i] = floatx4{q[0], q[1], q[2], q[3]};
        }
      } else {
        const int kk = k0 + kc[i];
        if (V && kk + 3 < K) {
          v[i] = *reinterpret_cast<const floatx4 *>(q);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[i][e] = (kk + e < K) ? q[e] : 0.0f;
        }
      }
    }
  }
};

// BK x COLS block, element (k, c) at X[k*ld + c], NT threads; vector i of
// thread t covers slab row (t + i*NT) / (COLS/4), block columns
// 4*((t + i*NT) % (COLS/4)) .. +3.  The row pointers advance by BK rows after
// every load.
template <int BK, int COLS, int NT, bool V>
struct KRowTileLoader {
  static constexpr int kVecs = BK * COLS / 4 / NT;
  static_assert((BK * COLS / 4) % NT == 0, "tile must split evenly over the threads");

  const float *ptr[kVecs];     // V: the 4-run itself; !V: start of the row
  int kr[kVecs];               // slab row
  int cols[V ? 1 : kVecs][4];  // !V: clamped column index of each element
  floatx4 v[kVecs];
  size_t step;                 // BK rows

  static __device__ __forceinline__ int row_of(int tid, int i) { return (tid + i * NT) / (COLS / 4); }
  static __device__ __forceinline__ int col_of(int tid, int i) { return ((tid + i * NT) % (COLS / 4)) * 4; }

  // X: the matrix, ld its leading dimension, ncols its row length (N or M),
  // c0 the block's first column.
  __device__ __forceinline__ void init(const float *X, int ld, int ncols, int c0, int tid) {
    step = (size_t)BK * (size_t)ld;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      kr[i] = row_of(tid, i);
      const int c = c0 + col_of(tid, i);
      if (V) {
        ptr[i] = X + (size_t)kr[i] * (size_t)ld + min(c, ncols - 4);
      } else {
        ptr[i] = X + (size_t)kr[i] * (size_t)ld;
#pragma unroll
        for (int e = 0; e < 4; ++e) cols[V ? 0 : i][e] = min(c + e, ncols - 1);
      }
    }
  }

  template <bool TAIL>
  __device__ __forceinline__ void load(int k0, int K) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      if (!TAIL || k0 + kr[i] < K) {
        if (V) {
          v[i] = *reinterpret_cast<const floatx4 *>(ptr[i]);
        } else {
          const float *q = ptr[i];
          v[i] = floatx4{q[cols[V ? 0 : i][0]], q[cols[V ? 0 : i][1]], q[cols[V ? 0 : i][2]],
                         q[cols[V ? 0 : i][3]]};
        }
      } else {
        v[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      ptr[i] += step;
    }
  }
};

}  // namespace sg950
