// sgemm_tiles.hpp -- global-memory loaders for one K-slab of the A and B tiles.
//
// A workgroup that owns a BM x BN tile of C walks K in slabs of BK: per slab
// it needs the BM x BK block of A (contiguous along K) and the BK x BN block of
// B (contiguous along N).  The threads read both with lanes running along the
// contiguous dimension, four floats per lane, so a 64-lane wavefront issues
// one 16-byte load per lane covering whole 64- to 256-byte row segments ("The
// road to a fast GEMM", sections "v0 to v1" and "v5: vectorized loads", on
// letting the lane index run along the contiguous dimension and on 128-bit
// accesses).
//
// Edges.  Rows of A past M and columns of B past N are clamped to the last
// valid row / column: those loads stay inside the matrix and only feed
// accumulators whose outputs are never stored.  K is different -- every k
// contributes to every output -- so in the last, partial slab the elements
// with k >= K are replaced by zero (selected, never multiplied, so a NaN or
// Inf in the matrix cannot leak in) and are not loaded at all.
//
// Alignment.  With V = true a lane loads its four floats as one 16-byte
// vector; that needs a 16-byte aligned base and a leading dimension that is a
// multiple of four (and, for B, N a multiple of four so a vector never crosses
// the end of a row).  With V = false the same four floats are loaded one by
// one, which works for any pointer and leading dimension.
#pragma once

#include "sgemm_common.hpp"

namespace sg950 {

// BM x BK block of A, NT threads; vector i of thread t covers tile row
// (t + i*NT) / (BK/4), tile columns 4*((t + i*NT) % (BK/4)) .. +3.
template <int BM, int BK, int NT, bool V>
struct ATileLoader {
  static constexpr int kVecs = BM * BK / 4 / NT;
  static_assert((BM * BK / 4) % NT == 0, "A tile must split evenly over the threads");
  static_assert(BK % 4 == 0, "BK must be a multiple of 4");

  const float *ptr[kVecs];  // element (row, 4-run start) at k = 0
  int kc[kVecs];            // k offset of the run inside the slab
  floatx4 v[kVecs];

  static __device__ __forceinline__ int row_of(int tid, int i) { return (tid + i * NT) / (BK / 4); }
  static __device__ __forceinline__ int col_of(int tid, int i) { return ((tid + i * NT) % (BK / 4)) * 4; }

  __device__ __forceinline__ void init(const Problem &p, int m0, int tid) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int row = min(m0 + row_of(tid, i), p.M - 1);
      kc[i] = col_of(tid, i);
      ptr[i] = p.A + (size_t)row * (size_t)p.lda + kc[i];
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

// BK x BN block of B, NT threads; vector i of thread t covers slab row
// (t + i*NT) / (BN/4), tile columns 4*((t + i*NT) % (BN/4)) .. +3.  The row
// pointers advance by BK rows after every load.
template <int BK, int BN, int NT, bool V>
struct BTileLoader {
  static constexpr int kVecs = BK * BN / 4 / NT;
  static_assert((BK * BN / 4) % NT == 0, "B tile must split evenly over the threads");

  const float *ptr[kVecs];  // V: the 4-run itself; !V: start of the row
  int kr[kVecs];            // slab row
  int cols[V ? 1 : kVecs][4];  // !V: clamped column index of each element
  floatx4 v[kVecs];
  size_t step;              // BK rows

  static __device__ __forceinline__ int row_of(int tid, int i) { return (tid + i * NT) / (BN / 4); }
  static __device__ __forceinline__ int col_of(int tid, int i) { return ((tid + i * NT) % (BN / 4)) * 4; }

  __device__ __forceinline__ void init(const Problem &p, int n0, int tid) {
    step = (size_t)BK * (size_t)p.ldb;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      kr[i] = row_of(tid, i);
      const int c = n0 + col_of(tid, i);
      if (V) {
        ptr[i] = p.B + (size_t)kr[i] * (size_t)p.ldb + min(c, p.N - 4);
      } else {
        ptr[i] = p.B + (size_t)kr[i] * (size_t)p.ldb;
#pragma unroll
        for (int e = 0; e < 4; ++e) cols[V ? 0 : i][e] = min(c + e, p.N - 1);
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
