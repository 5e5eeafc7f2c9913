// sgemm_valu.hip -- register-tiled SGEMM on the vector ALUs.
//
// The vector-ALU counterpart of the matrix-core kernel, following the ladder
// of "The road to a fast GEMM" (sections "v4: two-dimensional register
// tiling", "v5: vectorized loads" and the double-buffering exercise) and the
// tuning notes of the Tinyforge README (deeper K-slab, padded shared tile),
// re-shaped for gfx950:
//   * a 256-thread workgroup owns a 128 x 128 tile of C; each thread owns an
//     8 x 8 block of it, kept in 64 accumulator registers and updated as an
//     outer product: per k, 8 values of A and 8 of B feed 64 FMAs;
//   * both tiles are stored k-major in LDS (As[k][m], Bs[k][n]) so a thread's
//     8 A values are two 16-byte reads, like its 8 B values (an operand whose
//     memory rows run along K is transposed on its way into LDS);
//   * a thread's 8 rows are {4*ty .. 4*ty+3} and {64+4*ty .. 64+4*ty+3} (and
//     likewise its 8 columns), so the 16 lanes that read one LDS row at a time
//     touch 16 consecutive 16-byte chunks: no bank conflicts on the reads;
//   * two LDS buffers alternate with one barrier per K-slab of 16.
// Its ceiling is the plain v_fma_f32 rate (half the FP32 peak, which needs
// packed FMA; packed FP32 instructions are disabled in this build).
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_tiles.hpp"

#include <climits>
#include <type_traits>

namespace sg950 {

namespace {
constexpr int kBM = 128, kBN = 128, kBK = 16, kThreads = 256;
constexpr int kAPitch = kBM + 4;  // k-major A row pitch (floats)
constexpr int kBPitch = kBN + 4;  // B row pitch (floats)
}  // namespace

template <bool TA, bool TB, bool VA, bool VB, bool VC>
__global__ __launch_bounds__(kThreads) void valu_kernel(Problem p, int tiles_m, int tiles_n,
                                                        int group_m) {
  select_slice(p);
  __shared__ __attribute__((aligned(16))) float As[2 * kBK * kAPitch];
  __shared__ __attribute__((aligned(16))) float Bs[2 * kBK * kBPitch];

  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  const int tid = threadIdx.x;
  const int tx = tid & 15;
  const int ty = tid >> 4;

  // Both tiles live k-major in LDS (As[k][m], Bs[k][n]).  An operand whose
  // memory rows run along K (A untransposed, B transposed) is transposed on
  // the way in with four scalar stores per vector; the other kind is stored
  // as is.
  using LA = typename std::conditional<TA, KRowTileLoader<kBK, kBM, kThreads, VA>,
                                       RowTileLoader<kBM, kBK, kThreads, VA>>::type;
  using LB = typename std::conditional<TB, RowTileLoader<kBN, kBK, kThreads, VB>,
                                       KRowTileLoader<kBK, kBN, kThreads, VB>>::type;
  LA la;
  LB lb;
  la.init(p.A, p.lda, p.M, m0, tid);
  lb.init(p.B, p.ldb, p.N, n0, tid);

  // LDS store positions (k-major).
  int a_st[LA::kVecs];
  int b_st[LB::kVecs];
#pragma unroll
  for (int i = 0; i < LA::kVecs; ++i)
    a_st[i] = TA ? LA::row_of(tid, i) * kAPitch + LA::col_of(tid, i)
                 : LA::col_of(tid, i) * kAPitch + LA::row_of(tid, i);
#pragma unroll
  for (int i = 0; i < LB::kVecs; ++i)
    b_st[i] = TB ? LB::col_of(tid, i) * kBPitch + LB::row_of(tid, i)
                 : LB::row_of(tid, i) * kBPitch + LB::col_of(tid, i);

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;
  const bool ragged = (K % kBK) != 0;

  auto stage = [&](float *as, float *bs) {
#pragma unroll
    for (int i = 0; i < LA::kVecs; ++i) {
      if (TA) {
        *reinterpret_cast<floatx4 *>(as + a_st[i]) = la.v[i];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) as[a_st[i] + e * kAPitch] = la.v[i][e];
      }
    }
#pragma unroll
    for (int i = 0; i < LB::kVecs; ++i) {
      if (TB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[b_st[i] + e * kBPitch] = lb.v[i][e];
      } else {
        *reinterpret_cast<floatx4 *>(bs + b_st[i]) = lb.v[i];
      }
    }
  };

  if (ragged && nk == 1) {
    la.template load<true>(0, K);
    lb.template load<true>(0, K);
  } else {
    la.template load<false>(0, K);
    lb.template load<false>(0, K);
  }
  stage(As, Bs);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool has_next = kt + 1 < nk;
    if (has_next) {
      const int k1 = (kt + 1) * kBK;
      if (ragged && kt + 2 == nk) {
        la.template load<true>(k1, K);
        lb.template load<true>(k1, K);
      } else {
        la.template load<false>(k1, K);
        lb.template load<false>(k1, K);
      }
    }
    const float *as = As + cur * kBK * kAPitch + 4 * ty;
    const float *bs = Bs + cur * kBK * kBPitch + 4 * tx;
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const floatx4 a0 = *reinterpret_cast<const floatx4 *>(as + k * kAPitch);
      const floatx4 a1 = *reinterpret_cast<const floatx4 *>(as + k * kAPitch + 64);
      const floatx4 b0 = *reinterpret_cast<const floatx4 *>(bs + k * kBPitch);
      const floatx4 b1 = *reinterpret_cast<const floatx4 *>(bs + k * kBPitch + 64);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    if (has_next) stage(As + (cur ^ 1) * kBK * kAPitch, Bs + (cur ^ 1) * kBK * kBPitch);
    __syncthreads();
  }

  // Epilogue: rows 4*ty + {0..3} and 64 + 4*ty + {0..3}; columns likewise with
  // tx.  Whole in-range 4-column groups of an aligned C use 16-byte accesses.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
    if (row >= p.M) continue;
    float *crow = p.C + (size_t)row * (size_t)p.ldc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0 + h * 64 + 4 * tx;
      if (VC && col + 3 < p.N) {
        floatx4 *c4 = reinterpret_cast<floatx4 *>(crow + col);
        floatx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = p.alpha * acc[i][h * 4 + e];
        if (p.beta != 0.0f) {
          const floatx4 c = *c4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf(p.beta, c[e], o[e]);
        }
        *c4 = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < p.N) store_out(crow + col + e, acc[i][h * 4 + e], p.alpha, p.beta);
      }
    }
  }
}

template <bool TA, bool TB>
static void launch_valu_t(const Problem &p, dim3 grid, hipStream_t stream, int tm, int tn, int gm) {
  const bool va = a_vec_ok(p), vb = b_vec_ok(p), vc = c_vec_ok(p);
  const dim3 block(kThreads);
  // The C alignment only changes the epilogue, so it is folded into the
  // fully aligned case rather than doubling the instantiations.
  if (va && vb && vc) {
    SG950_LAUNCH((valu_kernel<TA, TB, true, true, true>), grid, block, 0, stream, p, tm, tn, gm);
  } else if (va && vb) {
    SG950_LAUNCH((valu_kernel<TA, TB, true, true, false>), grid, block, 0, stream, p, tm, tn, gm);
  } else if (va) {
    SG950_LAUNCH((valu_kernel<TA, TB, true, false, false>), grid, block, 0, stream, p, tm, tn, gm);
  } else if (vb) {
    SG950_LAUNCH((valu_kernel<TA, TB, false, true, false>), grid, block, 0, stream, p, tm, tn, gm);
  } else {
    SG950_LAUNCH((valu_kernel<TA, TB, false, false, false>), grid, block, 0, stream, p, tm, tn, gm);
  }
}

int launch_valu_128x128(const Problem &p, hipStream_t stream) {
  const long long tiles_m = ((long long)p.M + kBM - 1) / kBM;
  const long long tiles_n = ((long long)p.N + kBN - 1) / kBN;
  if (tiles_m * tiles_n > (long long)INT_MAX) return -1;
  const dim3 grid((unsigned)(tiles_m * tiles_n), 1, (unsigned)p.batch);
  const int tm = (int)tiles_m, tn = (int)tiles_n, gm = 8;
  if (!p.ta && !p.tb) {
    launch_valu_t<false, false>(p, grid, stream, tm, tn, gm);
  } else if (!p.ta) {
    launch_valu_t<false, true>(p, grid, stream, tm, tn, gm);
  } else if (!p.tb) {
    launch_valu_t<true, false>(p, grid, stream, tm, tn, gm);
  } else {
    launch_valu_t<true, true>(p, grid, stream, tm, tn, gm);
  }
  return 0;
}

}  // namespace sg950
