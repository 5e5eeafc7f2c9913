// sgemm_mfma.hpp -- strict-FP32 SGEMM on the CDNA4 matrix cores: the kernel
// template and its launch helpers (instantiated by sgemm_mfma.hip and
// sgemm_mfma8.hip).
//
// SGEMM is a dense contraction, so on gfx950 its inner product belongs on the
// matrix cores.  The instructions used take FP32 operands and accumulate in
// FP32 -- no input is rounded to a narrower format:
//   v_mfma_f32_32x32x2f32: a 32x32 block of C += (32x2 of A) x (2x32 of B)
//   v_mfma_f32_16x16x4f32: a 16x16 block of C += (16x4 of A) x (4x16 of B)
// Each is 64 FLOP per matrix-core clock per SIMD, the 157.3 TFLOP/s FP32
// peak of the datasheet (which the packed vector FMA shares).  Measured on
// MI355X: 155 TFLOP/s for 32x32x2, 141 for 16x16x4 in a plain chain, and 129
// for unpacked v_fma_f32 on the vector units.
//
// Structure (the tiling hierarchy of "The road to a fast GEMM", sections
// "v2: shared-memory tiling", "v4: two-dimensional register tiling" and "Where
// to go next" -- block tile, warp tile, matrix instruction -- re-sized for
// wave64 and the CDNA4 LDS):
//   * a workgroup owns a BM x BN tile of C and walks K in slabs of BK;
//   * its WAVES_M x WAVES_N wavefronts each own a (BM/WAVES_M) x (BN/WAVES_N)
//     wave tile, held as FM x FN matrix-core blocks in accumulator registers;
//   * each slab of A and B is read from global memory with 16-byte loads and
//     staged in LDS; two LDS buffers alternate so the global loads of slab
//     t+1 are in flight while slab t is multiplied, with one barrier per slab
//     (the double-buffering exercise of "The road to a fast GEMM").
//
// Operand layout.  For the 32x32x2 instruction lane l supplies A[l%32][k] and
// B[k][l%32] with k = l/32 (the 16x16x4 one: A[l%16][l/16], B[l/16][l%16]).
// Which k of the slab a lane group stands for is free, as long as A and B
// agree.  With the 32x32x2 instruction lane group g takes the KPG = BK/2
// consecutive k values [g*KPG, (g+1)*KPG); with the 16x16x4 one, whose four
// lane groups would otherwise read rows KPG apart -- a multiple of 64 banks
// for the padded M/N-contiguous tiles, a four-way conflict -- group g takes
// the runs of four k at 4g + 16q (q = 0, 1, ...), so the groups read rows four
// apart, on disjoint banks.  Each operand tile is kept in LDS in the
// orientation it has in memory:
//   * k contiguous (A untransposed, B transposed): rows of BK+4 floats; a
//     lane's four k values of an operand group are one 16-byte read, and the
//     4-float pad puts the reads of 8 (or 16) consecutive rows on disjoint
//     banks;
//   * M or N contiguous (B untransposed, A transposed): rows along k, padded
//     by 4 floats (BPAD for B); a lane reads its four k values as scalars, each
//     32-lane half reading 32 consecutive floats.
// With op(A), op(B) in {N, T} this gives the four transpose combinations from
// one kernel template.
//
// Output layout.  Lane l of a 32x32 block holds column l%32 and, in register
// r, row 8*(r/4) + 4*(l/32) + r%4; of a 16x16 block, row 4*(l/16) + r.
#pragma once

#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_tiles.hpp"

#include <climits>
#include <type_traits>

namespace sg950 {

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int BPAD, bool TA, bool TB>
struct MfmaTile {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M;  // wave tile rows
  static constexpr int WTN = BN / WAVES_N;  // wave tile columns
  static constexpr int FM = WTM / MI;       // matrix-core blocks per wave, M
  static constexpr int FN = WTN / MI;       // matrix-core blocks per wave, N
  static constexpr int KG = 64 / MI;        // lane groups along k
  static constexpr int KPG = BK / KG;       // k values per lane group and slab
  static constexpr int NQ = KPG / 4;        // 4-deep operand groups per slab
  // k of lane group g's first value (g * GK) and k distance between its
  // operand groups (QK): consecutive runs for 32x32x2, interleaved runs of
  // four for 16x16x4.
  static constexpr int GK = (MI == 16) ? 4 : KPG;
  static constexpr int QK = (MI == 16) ? 4 * KG : 4;
  // LDS row pitch (floats) and stage size of each operand tile.
  static constexpr int APITCH = TA ? BM + 4 : BK + 4;
  static constexpr int BPITCH = TB ? BK + 4 : BN + BPAD;
  static constexpr int A_STAGE = TA ? BK * APITCH : BM * APITCH;
  static constexpr int B_STAGE = TB ? BN * BPITCH : BK * BPITCH;
  static_assert(MI == 32 || MI == 16, "32x32x2 or 16x16x4 instruction");
  static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must hold whole blocks");
  static_assert(KPG % 4 == 0, "operands are read from LDS 4 k at a time");
  static_assert(BPAD % 4 == 0, "B rows must stay 16-byte aligned");
};

__device__ __forceinline__ floatx16 mfma_step(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_step(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row inside an MI x MI block of accumulator register r of lane group g.
template <int MI>
__device__ __forceinline__ int acc_row(int g, int r) {
  if constexpr (MI == 32) {
    return 8 * (r / 4) + 4 * g + (r % 4);
  } else {
    return 4 * g + r;
  }
}

// One 4-deep group of matrix-core operands of a wave: per MI-row block of
// op(A) and per MI-column block of op(B), four consecutive k.
template <class T>
struct Operands {
  floatx4 a[T::FM];
  floatx4 b[T::FN];
};

// Reads operand group q of a slab; `as` / `bs` already point at this lane's
// first A element and first B element in the stage.
template <int MI, bool TA, bool TB, class T>
__device__ __forceinline__ void read_operands(Operands<T> &o, const float *as, const float *bs, int q) {
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    if constexpr (!TA) {
      o.a[i] = *reinterpret_cast<const floatx4 *>(as + i * MI * T::APITCH + T::QK * q);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o.a[i][e] = as[(T::QK * q + e) * T::APITCH + i * MI];
    }
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    if constexpr (!TB) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o.b[j][e] = bs[(T::QK * q + e) * T::BPITCH + j * MI];
    } else {
      o.b[j] = *reinterpret_cast<const floatx4 *>(bs + j * MI * T::BPITCH + T::QK * q);
    }
  }
}

template <class T, class Acc>
__device__ __forceinline__ void multiply(Acc (&acc)[T::FM][T::FN], const Operands<T> &o) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = mfma_step(o.a[i][e], o.b[j][e], acc[i][j]);
}

// MINW is the minimum number of waves per SIMD the register allocation must
// leave room for (two waves per SIMD for the eight-wave 256x256 tile).
//
// Two LDS stages alternate: slab t+1 is loaded from global memory while slab
// t is multiplied and stored to the other stage after it; one barrier per
// slab.  With PIPE the order inside a slab is pinned by scheduling barriers:
// operand group q+1 is read before group q is multiplied, the next slab's
// registers are stored to the free stage in mid-slab, and the last group of a
// slab is multiplied after the barrier, behind the first reads of the next
// slab.  The store and that read are unconditional: on the last slab they only
// touch the stage nobody reads any more.  PIPE pays off on long K loops with
// 128x128 tiles; the plain order (left to the compiler, which interleaves the
// operand reads finely with the matrix instructions) is faster elsewhere.
//
// SPLITK: blockIdx.y selects a range of k_per_split values of K (a multiple
// of BK); the workgroup multiplies only that range and adds alpha times its
// partial product into C with float atomics (C was scaled by beta before the
// launch).  This fills the GPU when there are too few output tiles.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD, bool PIPE,
          bool SPLITK, bool TA, bool TB, bool VA, bool VB>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, MINW) void mfma_kernel(Problem p, int tiles_m,
                                                                              int tiles_n, int group_m,
                                                                              int k_per_split) {
  select_slice(p);
  if constexpr (SPLITK) {
    const int kb = blockIdx.y * k_per_split;  // < K by construction of the grid
    p.A += TA ? (size_t)kb * (size_t)p.lda : (size_t)kb;
    p.B += TB ? (size_t)kb : (size_t)kb * (size_t)p.ldb;
    p.K = min(p.K - kb, k_per_split);
  }
  using T = MfmaTile<MI, BM, BN, BK, WAVES_M, WAVES_N, BPAD, TA, TB>;
  using Acc = typename std::conditional<MI == 32, floatx16, floatx4>::type;
  constexpr int kRegs = MI * MI / 64;

  __shared__ __attribute__((aligned(16))) float As[2 * T::A_STAGE];
  __shared__ __attribute__((aligned(16))) float Bs[2 * T::B_STAGE];

  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int g = lane / MI;
  const int li = lane % MI;

  using LA = typename std::conditional<TA, KRowTileLoader<BK, BM, T::kThreads, VA>,
                                       RowTileLoader<BM, BK, T::kThreads, VA>>::type;
  using LB = typename std::conditional<TB, RowTileLoader<BN, BK, T::kThreads, VB>,
                                       KRowTileLoader<BK, BN, T::kThreads, VB>>::type;
  LA la;
  LB lb;
  la.init(p.A, p.lda, p.M, m0, tid);
  lb.init(p.B, p.ldb, p.N, n0, tid);

  Acc acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < kRegs; ++r) acc[i][j][r] = 0.0f;

  const int K = p.K;
  const int nk = (K + BK - 1) / BK;
  const bool ragged = (K % BK) != 0;

  // LDS offsets of this thread's stores and of its wave's operand reads.
  int a_st[LA::kVecs];
  int b_st[LB::kVecs];
#pragma unroll
  for (int i = 0; i < LA::kVecs; ++i) a_st[i] = LA::row_of(tid, i) * T::APITCH + LA::col_of(tid, i);
#pragma unroll
  for (int i = 0; i < LB::kVecs; ++i) b_st[i] = LB::row_of(tid, i) * T::BPITCH + LB::col_of(tid, i);
  const int a_rd = TA ? (g * T::GK) * T::APITCH + wm * T::WTM + li
                      : (wm * T::WTM + li) * T::APITCH + g * T::GK;
  const int b_rd = TB ? (wn * T::WTN + li) * T::BPITCH + g * T::GK
                      : (g * T::GK) * T::BPITCH + wn * T::WTN + li;

  // Loads slab `slab` into the loaders' registers (zero-filled K tail).
  auto load = [&](int slab) {
    const int k0 = slab * BK;
    if (ragged && slab == nk - 1) {
      la.template load<true>(k0, K);
      lb.template load<true>(k0, K);
    } else {
      la.template load<false>(k0, K);
      lb.template load<false>(k0, K);
    }
  };
  auto store = [&](int stage) {
    float *an = As + stage * T::A_STAGE;
    float *bn = Bs + stage * T::B_STAGE;
#pragma unroll
    for (int i = 0; i < LA::kVecs; ++i) *reinterpret_cast<floatx4 *>(an + a_st[i]) = la.v[i];
#pragma unroll
    for (int i = 0; i < LB::kVecs; ++i) *reinterpret_cast<floatx4 *>(bn + b_st[i]) = lb.v[i];
  };

  load(0);
  store(0);
  __syncthreads();
  if constexpr (PIPE) {
    Operands<T> o;
    read_operands<MI, TA, TB>(o, As + a_rd, Bs + b_rd, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
      const float *as = As + cur * T::A_STAGE + a_rd;
      const float *bs = Bs + cur * T::B_STAGE + b_rd;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q + 1 < T::NQ; ++q) {
        Operands<T> nxt;
        read_operands<MI, TA, TB>(nxt, as, bs, q + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (q == T::NQ / 2 - 1) {
          store(cur ^ 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        multiply<T>(acc, o);
        o = nxt;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (T::NQ == 1) store(cur ^ 1);
      __syncthreads();
      Operands<T> nxt;
      read_operands<MI, TA, TB>(nxt, As + (cur ^ 1) * T::A_STAGE + a_rd,
                                Bs + (cur ^ 1) * T::B_STAGE + b_rd, 0);
      __builtin_amdgcn_sched_barrier(0);
      multiply<T>(acc, o);
      o = nxt;
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool has_next = kt + 1 < nk;
      if (has_next) load(kt + 1);
      const float *as = As + cur * T::A_STAGE + a_rd;
      const float *bs = Bs + cur * T::B_STAGE + b_rd;
#pragma unroll
      for (int q = 0; q < T::NQ; ++q) {
        Operands<T> o;
        read_operands<MI, TA, TB>(o, as, bs, q);
        multiply<T>(acc, o);
      }
      if (has_next) store(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: C = alpha*acc + beta*C for the in-range elements.  For a fixed
  // register, the MI lanes of a group write MI consecutive floats of one row.
  const int row0 = m0 + wm * T::WTM;
  const int col0 = n0 + wn * T::WTN + li;
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int col = col0 + j * MI;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < kRegs; ++r) {
        const int row = row0 + i * MI + acc_row<MI>(g, r);
        if (row >= p.M) continue;
        float *c = p.C + (size_t)row * (size_t)p.ldc + col;
        if constexpr (SPLITK) {
          atomicAdd(c, p.alpha * acc[i][j][r]);
        } else {
          store_out(c, acc[i][j][r], p.alpha, p.beta);
        }
      }
    }
}

// Number of K splits for a grid of `tiles` output tiles (over all batch
// slices): none when the tiles
// alone give every CU a workgroup, otherwise enough for about two workgroups
// per CU, each split at least four slabs deep.
template <int BK>
static int choose_splits(long long tiles, int K, int &k_per_split) {
  const long long cus = 256, target = 512;
  long long splits = (tiles >= cus) ? 1 : (target + tiles - 1) / tiles;
  const long long max_splits = K / (4 * BK);
  if (splits > max_splits) splits = max_splits;
  if (splits < 2) {
    k_per_split = K;
    return 1;
  }
  long long kps = ((long long)K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  k_per_split = (int)kps;
  return (int)(((long long)K + kps - 1) / kps);
}

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD, bool PIPE,
          bool SPLITK, bool TA, bool TB>
static void launch_mfma_aligned(const Problem &p, dim3 grid, dim3 block, hipStream_t stream, int tm,
                                int tn, int group_m, int k_per_split) {
  const bool va = a_vec_ok(p), vb = b_vec_ok(p);
#define SG950_LAUNCH_VA(VA_, VB_)                                                                     \
  SG950_LAUNCH(                                                                                \
      (mfma_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, PIPE, SPLITK, TA, TB, VA_, VB_>), \
      grid, block, 0, stream, p, tm, tn, group_m, k_per_split)
  if (va && vb) {
    SG950_LAUNCH_VA(true, true);
  } else if (va) {
    SG950_LAUNCH_VA(true, false);
  } else if (vb) {
    SG950_LAUNCH_VA(false, true);
  } else {
    SG950_LAUNCH_VA(false, false);
  }
#undef SG950_LAUNCH_VA
}

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD, bool PIPE,
          bool SPLITK>
static void launch_mfma_split(const Problem &p, dim3 grid, dim3 block, hipStream_t stream, int tm,
                              int tn, int group_m, int k_per_split) {
#define SG950_LAUNCH_T(TA_, TB_)                                                                 \
  launch_mfma_aligned<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, PIPE, SPLITK, TA_, TB_>(p, grid, \
      block, stream, tm, tn, group_m, k_per_split)
  if (!p.ta && !p.tb) {
    SG950_LAUNCH_T(false, false);
  } else if (!p.ta) {
    SG950_LAUNCH_T(false, true);
  } else if (!p.tb) {
    SG950_LAUNCH_T(true, false);
  } else {
    SG950_LAUNCH_T(true, true);
  }
#undef SG950_LAUNCH_T
}

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD, bool PIPE,
          bool SPLITK>
static int launch_mfma(const Problem &p, hipStream_t stream) {
  const long long tiles_m = ((long long)p.M + BM - 1) / BM;
  const long long tiles_n = ((long long)p.N + BN - 1) / BN;
  if (tiles_m * tiles_n > (long long)INT_MAX) return -1;
  int k_per_split = p.K;
  const int splits = SPLITK ? choose_splits<BK>(tiles_m * tiles_n * p.batch, p.K, k_per_split) : 1;
  if (SPLITK && splits > 1) {
    if (splits > 65535) return -1;
    // C = beta*C first; the split workgroups then add into it.
    if (p.beta != 1.0f && launch_scale(p, stream) != 0) return -1;
  }
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits, (unsigned)p.batch);
  const dim3 block(WAVES_M * WAVES_N * 64);
  const int tm = (int)tiles_m, tn = (int)tiles_n, group_m = 8;
  if (SPLITK && splits > 1) {
    launch_mfma_split<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, PIPE, SPLITK>(
        p, grid, block, stream, tm, tn, group_m, k_per_split);
  } else {
    launch_mfma_split<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, PIPE, false>(
        p, grid, block, stream, tm, tn, group_m, k_per_split);
  }
  return 0;
}

#define SG950_MFMA_LAUNCHER(name, MI, BM, BN, BK, WM, WN, MINW, BPAD, PIPE, SPLITK) \
  int launch_##name(const Problem &p, hipStream_t s) {                              \
    return launch_mfma<MI, BM, BN, BK, WM, WN, MINW, BPAD, PIPE, SPLITK>(p, s);     \
  }

}  // namespace sg950
