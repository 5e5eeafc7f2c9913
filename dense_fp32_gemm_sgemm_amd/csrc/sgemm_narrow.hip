// sgemm_narrow.hip -- SGEMM with few columns of C (N <= 16): a product bound
// by the bandwidth of streaming A.
//
// With N <= 16 a GEMM does at most 32 FLOP per element of A it reads, near or
// below the MI355X ridge point: A has to stream from HBM once, and the kernel
// keeps many loads in flight without staging A in LDS.
//
// A workgroup owns 16 rows of C and runs the whole K with eight waves, wave w
// taking the w-th of eight contiguous K ranges.  Each wave accumulates its
// 16 x 16 block of C on the matrix cores with v_mfma_f32_16x16x4f32 (lane l
// supplies A[l%16][k] and B[k][l%16], lane group g = l/16 standing for the
// runs of four k at 16q + 4g, as in the tiled kernels): per group of 16 k a
// lane loads one 16-byte vector of its row of A straight from global memory
// and four values of its column of B (16 lanes read 64 consecutive bytes of a
// row of B, which stays in L2), and issues four matrix instructions.  Eight
// groups of loads are issued before their first use.  Columns past N read
// column N-1 and rows past M read row M-1 (in bounds, never stored); k past K
// in the last group is skipped by selection, so a NaN or Inf outside the
// matrices cannot leak in.  The eight waves' blocks are added through LDS in
// a fixed order and C = alpha*sum + beta*C is written once: one launch, no
// atomics, deterministic.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"

#include <climits>

namespace sg950 {

namespace {
constexpr int kNarrowRows = 16;   // rows of C per workgroup
constexpr int kNarrowCols = 16;   // columns of C (N <= 16)
constexpr int kNarrowWaves = 8;   // waves per workgroup, each a K range
constexpr int kNarrowUnroll = 8;  // groups of 16 k whose loads are in flight
}  // namespace

// VA: A untransposed, its rows read as 16-byte vectors along K.
// VB: B transposed (stored N x K), its rows read as 16-byte vectors along K.
// The vectors go through copies that need only 4-byte alignment, which a
// global load of 16 bytes also needs: a leading dimension that is not a
// multiple of 4 keeps them (four single loads instead stream A at about
// half the rate).
template <bool TA, bool TB, bool VA, bool VB>
__global__ __launch_bounds__(kNarrowWaves * 64) void narrow_kernel(Problem p, int krange) {
  select_slice(p);
  __shared__ floatx4 red[kNarrowWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane % 16, g = lane / 16;
  const int row = min((int)blockIdx.x * kNarrowRows + li, p.M - 1);  // A row of this lane
  const int col = min(li, p.N - 1);                                    // B column of this lane
  const int kb = w * krange;                    // this wave's K range [kb, ke)
  const int ke = min(p.K, kb + krange);
  const size_t lda = (size_t)p.lda, ldb = (size_t)p.ldb;

  // Four consecutive k of this lane's row of op(A), and of its column of op(B).
  auto load_a = [&](int k) -> floatx4 {
    if constexpr (!TA && VA) {
      floatx4 v;
      __builtin_memcpy(&v, p.A + (size_t)row * lda + k, sizeof(v));
      return v;
    } else if constexpr (!TA) {
      const float *q = p.A + (size_t)row * lda + k;
      return floatx4{q[0], q[1], q[2], q[3]};
    } else {
      const float *q = p.A + (size_t)k * lda + row;
      return floatx4{q[0], q[lda], q[2 * lda], q[3 * lda]};
    }
  };
  auto load_b = [&](int k) -> floatx4 {
    if constexpr (TB && VB) {
      floatx4 v;
      __builtin_memcpy(&v, p.B + (size_t)col * ldb + k, sizeof(v));
      return v;
    } else if constexpr (TB) {
      const float *q = p.B + (size_t)col * ldb + k;
      return floatx4{q[0], q[1], q[2], q[3]};
    } else {
      const float *q = p.B + (size_t)k * ldb + col;
      return floatx4{q[0], q[ldb], q[2 * ldb], q[3 * ldb]};
    }
  };

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // Groups of 16 k: lane group g takes k = k0 + 4g .. k0 + 4g + 3.
  const int nfull = (ke > kb) ? (ke - kb) / 16 : 0;  // groups inside [kb, ke)
  int t = 0;
  for (; t + kNarrowUnroll <= nfull; t += kNarrowUnroll) {
    floatx4 a[kNarrowUnroll], b[kNarrowUnroll];
#pragma unroll
    for (int u = 0; u < kNarrowUnroll; ++u) {
      const int k = kb + (t + u) * 16 + 4 * g;
      a[u] = load_a(k);
      b[u] = load_b(k);
    }
    // All loads of the batch are issued before the first use.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kNarrowUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][e], b[u][e], acc, 0, 0, 0);
  }
  for (; t < nfull; ++t) {
    const int k = kb + t * 16 + 4 * g;
    const floatx4 a = load_a(k), b = load_b(k);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }
  // The rest of the range (fewer than 16 k): element by element, k < ke only.
  const int kt = kb + nfull * 16;
  if (kt < ke) {
    floatx4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = kt + 4 * g + e;
      const bool in = k < ke;
      const int kk = in ? k : kb;  // any in-range k; the value is replaced below
      const float av = TA ? p.A[(size_t)kk * lda + row] : p.A[(size_t)row * lda + kk];
      const float bv = TB ? p.B[(size_t)col * ldb + kk] : p.B[(size_t)kk * ldb + col];
      a[e] = in ? av : 0.0f;
      b[e] = in ? bv : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }

  // Lane l holds column l%16 and rows 4*(l/16) + r of the 16 x 16 block.
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;  // no barrier after this point
  floatx4 s = red[0][lane];
#pragma unroll
  for (int q = 1; q < kNarrowWaves; ++q) {
    const floatx4 v = red[q][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] += v[r];
  }
  if (li >= p.N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int orow = (int)blockIdx.x * kNarrowRows + 4 * g + r;
    if (orow < p.M) store_out(p.C + (size_t)orow * (size_t)p.ldc + li, s[r], p.alpha, p.beta);
  }
}

namespace {
template <bool TA, bool TB>
void launch_narrow_t(const Problem &p, dim3 grid, hipStream_t stream, int krange) {
  const dim3 block(kNarrowWaves * 64);
  // 16-byte loads along K at any 4-byte aligned address.
  const bool va = !TA && (reinterpret_cast<uintptr_t>(p.A) & 3) == 0;
  const bool vb = TB && (reinterpret_cast<uintptr_t>(p.B) & 3) == 0;
  if (va && vb) {
    SG950_LAUNCH((narrow_kernel<TA, TB, true, true>), grid, block, 0, stream, p, krange);
  } else if (va) {
    SG950_LAUNCH((narrow_kernel<TA, TB, true, false>), grid, block, 0, stream, p, krange);
  } else if (vb) {
    SG950_LAUNCH((narrow_kernel<TA, TB, false, true>), grid, block, 0, stream, p, krange);
  } else {
    SG950_LAUNCH((narrow_kernel<TA, TB, false, false>), grid, block, 0, stream, p, krange);
  }
}
}  // namespace

int launch_narrow(const Problem &p, hipStream_t stream) {
  if (p.N > kNarrowCols) return -1;
  const long long blocks = ((long long)p.M + kNarrowRows - 1) / kNarrowRows;
  if (blocks > INT_MAX) return -1;
  // Eight K ranges, each a multiple of 16 (so groups stay 4-aligned).
  int krange = (p.K + kNarrowWaves - 1) / kNarrowWaves;
  krange = (krange + 15) / 16 * 16;
  const dim3 grid((unsigned)blocks, 1u, (unsigned)p.batch);
  if (!p.ta && !p.tb) {
    launch_narrow_t<false, false>(p, grid, stream, krange);
  } else if (!p.ta) {
    launch_narrow_t<false, true>(p, grid, stream, krange);
  } else if (!p.tb) {
    launch_narrow_t<true, false>(p, grid, stream, krange);
  } else {
    launch_narrow_t<true, true>(p, grid, stream, krange);
  }
  return 0;
}

}  // namespace sg950
