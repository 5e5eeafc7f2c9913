// sgemm_valu.hip -- register-tiled SGEMM on the vector ALUs.
//
// The vector-ALU counterpart of the matrix-core kernel, following the ladder
// of "The road to a fast GEMM" (sections "v4: two-dimensional register
// tiling", "v5: vectorized loads" and the double-buffering exercise) and the
// tuning notes of the Tinyforge README (register tiling as the main step,
// a deeper K-slab, a padded shared tile), re-shaped for gfx950:
//   * a 256-thread workgroup owns a 128 x 256 tile of C; each thread owns an
//     8 x 16 block of it in 128 accumulator registers, updated as an outer
//     product: per k, 8 values of A and 16 of B feed 128 FMAs;
//   * both tiles are stored k-major in LDS (As[k][m], Bs[k][n]) so a thread's
//     8 A values are two 16-byte reads and its 16 B values four (an operand
//     whose memory rows run along K is transposed on its way into LDS);
//   * a thread's 8 rows are {4*ty .. 4*ty+3} and {64+4*ty .. 64+4*ty+3} and
//     its 16 columns {4*tx + 64*c .. +3} (c = 0..3), so the 16 lanes that
//     read one LDS row at a time touch 16 consecutive 16-byte chunks: no bank
//     conflicts on the reads;
//   * two LDS buffers alternate with one barrier per K-slab of 16; the global
//     loads of the next slab are in flight while this one is multiplied, and
//     a ragged last slab is the only one that checks k against K.
// Why 8 x 16: LDS returns 128 bytes per clock to a CU, and every FMA needs
// its operands from LDS once per k.  An 8 x 8 block reads (8 + 8) * 4 bytes
// per 64 FMAs, 1 byte per lane-FMA -- at the measured vector FMA rate of
// gfx950 (about 105 lane-FMAs per clock per CU, 129 TFLOP/s with unpacked
// v_fma_f32) that is 82% of the LDS bandwidth; 8 x 16 needs 0.75 bytes, and
// the 128 accumulators still leave room for two workgroups per CU.
// Ceiling: the unpacked v_fma_f32 rate (packed FP32 instructions are switched
// off in the library's compile flags); the matrix cores, at 155 TFLOP/s measured for FP32,
// are the main path.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_tiles.hpp"

#include <climits>
#include <type_traits>

namespace sg950 {

namespace {
constexpr int kBM = 128, kBN = 256, kBK = 16, kThreads = 256;
constexpr int kTM = 8, kTN = 16;      // outputs per thread
constexpr int kAPitch = kBM + 4;      // k-major A row pitch (floats)
constexpr int kBPitch = kBN + 4;      // B row pitch (floats)
}  // namespace

template <bool TA, bool TB, bool VA, bool VB, bool VC>
__global__ __launch_bounds__(kThreads, 2) void valu_kernel(Problem p, int tiles_m, int tiles_n,
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

  float acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;
  const int nfull = K / kBK;  // slabs that lie wholly inside K

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
  auto load = [&](int kt) {
    if (kt < nfull) {
      la.template load<false>(kt * kBK, K);
      lb.template load<false>(kt * kBK, K);
    } else {
      la.template load<true>(kt * kBK, K);
      lb.template load<true>(kt * kBK, K);
    }
  };
  // The outer products of one slab from LDS stage `cur`.  The operands of
  // step k+1 are read while step k is multiplied, and a scheduling fence
  // after every step keeps the compiler from hoisting the reads of further
  // steps (which would need more registers than the accumulators leave).
  auto read_ops = [&](const float *as, const float *bs, int k, float (&a)[kTM], float (&b)[kTN]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const floatx4 v = *reinterpret_cast<const floatx4 *>(as + k * kAPitch + 64 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * h + e] = v[e];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const floatx4 v = *reinterpret_cast<const floatx4 *>(bs + k * kBPitch + 64 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) b[4 * c + e] = v[e];
    }
  };
  auto multiply = [&](int cur) {
    const float *as = As + cur * kBK * kAPitch + 4 * ty;
    const float *bs = Bs + cur * kBK * kBPitch + 4 * tx;
    float a[kTM], b[kTN];
    read_ops(as, bs, 0, a, b);
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      float an[kTM], bn[kTN];
      if (k + 1 < kBK) read_ops(as, bs, k + 1, an, bn);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      if (k + 1 < kBK) {
#pragma unroll
        for (int i = 0; i < kTM; ++i) a[i] = an[i];
#pragma unroll
        for (int j = 0; j < kTN; ++j) b[j] = bn[j];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load(0);
  stage(As, Bs);
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int cur = kt & 1;
    load(kt + 1);  // in flight while this slab is multiplied
    multiply(cur);
    stage(As + (cur ^ 1) * kBK * kAPitch, Bs + (cur ^ 1) * kBK * kBPitch);
    __syncthreads();
  }
  multiply((nk - 1) & 1);

  // Epilogue: rows 4*ty + {0..3} and 64 + 4*ty + {0..3}; columns 4*tx + 64*c
  // + {0..3}.  Whole in-range 4-column groups of an aligned C use 16-byte
  // accesses.
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
    if (row >= p.M) continue;
    float *crow = p.C + (size_t)row * (size_t)p.ldc;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
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

int launch_valu_128x256(const Problem &p, hipStream_t stream) {
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
