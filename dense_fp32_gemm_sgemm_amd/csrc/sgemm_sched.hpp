// sgemm_sched.hpp -- the matrix-core kernel with an explicitly ordered slab
// loop, for problems that span at least one tile in each dimension.
//
// It computes what mfma_kernel (sgemm_mfma.hpp) computes, with the same LDS
// layout, operand reads and matrix-core blocks, and (when BK divides K) the
// same order of the K-sum for every output.  The loop around them is
// different: the pages' double buffering ("The road to a fast GEMM", section
// on prefetching the next tile while computing the current one) is taken one
// step further, and the instruction order inside a slab is pinned instead of
// left to the compiler:
//
//   * operand group q+1 of the slab is read from LDS while group q is
//     multiplied, and those reads are issued first in the group, so they have
//     landed long before their matrix instructions;
//   * in the middle of slab t the registers holding slab t+1 are stored to the
//     free LDS stage and the global loads of slab t+2 are issued at once, two
//     matrix instructions apart: global loads get about a slab and a half to
//     arrive, with one set of staging registers;
//   * the last operand group of a slab is multiplied half before and half
//     after the barrier, behind the first LDS reads of the next slab;
//   * there are no branches in the slab loop: at the end the loads repeat the
//     last slab (clamped index) and the stores go to the stage nobody reads.
//
// K need not be a multiple of BK: every slab after the first then starts ov =
// nk*BK - K values of k early, so the last one ends at K and every load stays
// inside the operands, and the first slab's last ov values are overwritten
// with zeros in LDS, in both operands, so nothing is counted twice and no
// 0 * Inf arises.
//
// B operand reads.  With B untransposed (k-rows in LDS) and two or four
// matrix-core blocks across a wave tile, lane li of block j takes column
// FN*li + j of the wave tile instead of j*MI + li: its FN values of one k are
// then one 8- or 16-byte LDS read instead of FN scalar reads, and in the
// epilogue it holds FN consecutive columns of a row, written as one vector.
// The K-sum of every output is unchanged.
//
// Addressing is stateless: one base pointer per operand and thread, plus
// offsets that are uniform across the workgroup, which keeps the register
// count low enough for four waves with 128x128 wave tiles.  A tile that would
// stick out of C is shifted back inside (its first row becomes M - BM, or its
// first column N - BN), so every load is in bounds without clamping; the
// epilogue then stores only the rows and columns that belong to the tile.
//
// Global loads are 16-byte vectors of four consecutive floats; the hardware
// needs only 4-byte alignment for them, so leading dimensions, batch strides
// and shifted tiles may put them anywhere.
//
// K may also be split over workgroups (SPLITK, blockIdx.y): each range runs
// the same loop and adds its partial tile into C with atomics.
//
// Preconditions (checked on the host; other problems go to mfma_kernel):
// K >= BK, M >= BM (or, with SHORTM and A not transposed, M >= 1), N >= BN,
// A and B 4-byte aligned.
#pragma once

#include "sgemm_mfma.hpp"

namespace sg950 {

template <class T, class Acc, int E0, int E1>
__device__ __forceinline__ void multiply_part(Acc (&acc)[T::FM][T::FN], const Operands<T> &o) {
#pragma unroll
  for (int e = E0; e < E1; ++e)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = mfma_step(o.a[i][e], o.b[j][e], acc[i][j]);
}

// Stateless loader of one operand's slab: ROWS x BK (k contiguous, KROWS =
// false) or BK x ROWS (k-rows, KROWS = true) of a row-major matrix X with
// leading dimension ld.  Thread t handles the 4-float vectors t, t+NT, ...;
// with NT a multiple of the vectors per row, a thread's vectors sit at fixed
// uniform row distances (DR) in one column.
template <int ROWS, int BK, int NT, bool KROWS>
struct SlabLoader {
  static constexpr int COLS = KROWS ? ROWS : BK;  // floats per block row
  static constexpr int VPR = COLS / 4;           // vectors per block row
  static constexpr int NV = ROWS * BK / 4 / NT;  // vectors per thread
  static constexpr int DR = NT / VPR;            // block rows between them
  static_assert(NT % VPR == 0, "a thread's vectors must share one column");
  static_assert(ROWS * BK / 4 % NT == 0, "slab must split evenly over the threads");

  const float *base;  // this thread's first vector at k = 0
  size_t ld;
  int kpos;           // k of this thread's first value inside a slab
  floatx4 v[NV];

  // r0: first row (or column, for k-rows) of the block inside X.
  __device__ __forceinline__ void init(const float *X, int ld_, int r0, int tid) {
    ld = (size_t)ld_;
    const int br = tid / VPR, bc = (tid % VPR) * 4;
    base = KROWS ? X + (size_t)br * ld + r0 + bc : X + (size_t)(r0 + br) * ld + bc;
    kpos = KROWS ? br : bc;
  }

  // Writes zeros over this thread's values of a stored slab whose k inside
  // the slab is kcut or more (lds: the thread's vector 0 in the stage, pitch:
  // the stage's row pitch).
  __device__ __forceinline__ void zero_from(float *lds, int pitch, int kcut) const {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = KROWS ? kpos + i * DR : kpos + e;
        if (k >= kcut) lds[i * DR * pitch + e] = 0.0f;
      }
  }
  // Moves every later load d values of k back.
  __device__ __forceinline__ void shift_k(int d) { base -= KROWS ? (size_t)d * ld : (size_t)d; }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float *q = KROWS ? base + ((size_t)k0 + (size_t)i * DR) * ld
                             : base + (size_t)i * DR * ld + k0;
      // Four consecutive floats at any 4-byte aligned address: the copy
      // compiles to one global_load_dwordx4, which needs only dword alignment.
      floatx4 t;
      __builtin_memcpy(&t, q, sizeof(t));
      v[i] = t;
    }
  }
  // LDS offset (floats) of vector 0 in a stage of row pitch `pitch`; vector i
  // is i*DR rows further.
  static __device__ __forceinline__ int lds_offset(int tid, int pitch) {
    return (tid / VPR) * pitch + (tid % VPR) * 4;
  }
};

// SlabLoader for a row slab (k contiguous) that may extend past the last row
// of X: rows from `maxrow` on read row `maxrow` (never stored).  Each vector
// keeps its own row pointer.
template <int ROWS, int BK, int NT>
struct ClampedRowLoader : SlabLoader<ROWS, BK, NT, false> {
  using Base = SlabLoader<ROWS, BK, NT, false>;
  using Base::DR;
  using Base::NV;
  using Base::VPR;
  const float *rowp[NV];  // each vector's row at k = 0

  __device__ __forceinline__ void init(const float *X, int ld_, int r0, int tid, int maxrow) {
    this->ld = (size_t)ld_;
    const int br = tid / VPR, bc = (tid % VPR) * 4;
#pragma unroll
    for (int i = 0; i < NV; ++i) rowp[i] = X + (size_t)min(r0 + br + i * DR, maxrow) * this->ld + bc;
    this->kpos = bc;
  }
  __device__ __forceinline__ void shift_k(int d) {
#pragma unroll
    for (int i = 0; i < NV; ++i) rowp[i] -= d;
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      floatx4 t;
      __builtin_memcpy(&t, rowp[i] + k0, sizeof(t));
      this->v[i] = t;
    }
  }
};

// Operand reads of the ordered loop: as read_operands, except that with
// PERMB the B values of one k for the FN blocks are one vector read.
template <int MI, bool TA, bool TB, bool PERMB, class T>
__device__ __forceinline__ void read_sched_operands(Operands<T> &o, const float *as, const float *bs,
                                                    int q) {
  if constexpr (!PERMB) {
    read_operands<MI, TA, TB>(o, as, bs, q);
  } else {
    static_assert(!TB && (T::FN == 2 || T::FN == 4), "permuted B needs k-rows and 2 or 4 blocks");
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
    for (int e = 0; e < 4; ++e) {
      const float *row = bs + (T::QK * q + e) * T::BPITCH;
      if constexpr (T::FN == 4) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(row);
#pragma unroll
        for (int j = 0; j < 4; ++j) o.b[j][e] = v[j];
      } else {
        const floatx2 v = *reinterpret_cast<const floatx2 *>(row);
        o.b[0][e] = v[0];
        o.b[1][e] = v[1];
      }
    }
  }
}

// SPLITK: blockIdx.y selects a range of k_per_split values of K (the last
// range takes the rest, at least BK); the workgroup multiplies only that
// range and adds alpha times its partial product into C with float atomics
// (C was scaled by beta before the launch).
//
// SHORTM (A not transposed): M may be below BM; the tile then starts at row 0,
// rows from M on read row M - 1 of A and are not stored.
//
// TAIL (one batch slice): workgroups from tl.dp_tiles on each take one K
// range of a tile of the last round (TailArgs); the partial tiles meet in a
// fixed order, so the result does not depend on which range finishes last.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD, bool TA,
          bool TB, bool RAGGED, bool SPLITK, bool SHORTM = false, bool TAIL = false>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, MINW) void sched_kernel(Problem p, int tiles_m,
                                                                               int tiles_n, int group_m,
                                                                               int k_per_split,
                                                                               TailArgs tl) {
  static_assert(!(TAIL && (SPLITK || SHORTM)), "the tail form is its own split");
  select_slice(p);
  if constexpr (SPLITK) {
    const int kb = (int)blockIdx.y * k_per_split;
    p.A += TA ? (size_t)kb * (size_t)p.lda : (size_t)kb;
    p.B += TB ? (size_t)kb : (size_t)kb * (size_t)p.ldb;
    p.K = (blockIdx.y + 1 == gridDim.y) ? p.K - kb : k_per_split;
  }
  using T = MfmaTile<MI, BM, BN, BK, WAVES_M, WAVES_N, BPAD, TA, TB>;
  using Acc = typename std::conditional<MI == 32, floatx16, floatx4>::type;
  constexpr int kRegs = MI * MI / 64;
  constexpr int NT = T::kThreads;
  static_assert(T::NQ >= 2, "at least two operand groups per slab");
  constexpr bool CLAMPM = SHORTM && !TA;  // rows of A clamped (M < BM allowed)
  using LA = typename std::conditional<CLAMPM, ClampedRowLoader<BM, BK, NT>, SlabLoader<BM, BK, NT, TA>>::type;
  using LB = SlabLoader<BN, BK, NT, !TB>;
  constexpr bool PERMB = !TB && (T::FN == 2 || T::FN == 4);

  __shared__ __attribute__((aligned(16))) float As[2 * T::A_STAGE];
  __shared__ __attribute__((aligned(16))) float Bs[2 * T::B_STAGE];

  int tm, tn;
  int tail_t = -1, sidx = 0;  // TAIL: tile of the last round and K range, or -1 (whole tile)
  if constexpr (TAIL) {
    const int b = (int)blockIdx.x;
    int id;
    if (b < tl.dp_tiles) {
      id = xcd_remap(b, tl.dp_tiles);
    } else {
      const int j = b - tl.dp_tiles;
      tail_t = j / tl.splits;
      sidx = j - tail_t * tl.splits;
      id = tl.dp_tiles + tail_t;
      const int nkf = p.K / BK;  // whole slabs; the last range also takes the rest
      const int kb = (int)((long long)sidx * nkf / tl.splits) * BK;
      const int ke = (sidx + 1 == tl.splits) ? p.K : (int)((long long)(sidx + 1) * nkf / tl.splits) * BK;
      p.A += TA ? (size_t)kb * (size_t)p.lda : (size_t)kb;
      p.B += TB ? (size_t)kb : (size_t)kb * (size_t)p.ldb;
      p.K = ke - kb;
    }
    grouped_tile(id, tiles_m, tiles_n, group_m, tm, tn);
  } else {
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  // shifted inside C (with CLAMPM and M < BM: from row 0)
  const int ms = CLAMPM ? max(0, min(m0, p.M - BM)) : min(m0, p.M - BM), ns = min(n0, p.N - BN);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int g = lane / MI, li = lane % MI;

  LA la;
  LB lb;
  if constexpr (CLAMPM)
    la.init(p.A, p.lda, ms, tid, p.M - 1);
  else
    la.init(p.A, p.lda, ms, tid);
  lb.init(p.B, p.ldb, ns, tid);
  const int a_st = LA::lds_offset(tid, T::APITCH);
  const int b_st = LB::lds_offset(tid, T::BPITCH);
  auto store = [&](int stage) {
    float *an = As + stage * T::A_STAGE + a_st;
    float *bn = Bs + stage * T::B_STAGE + b_st;
#pragma unroll
    for (int i = 0; i < LA::NV; ++i) *reinterpret_cast<floatx4 *>(an + i * LA::DR * T::APITCH) = la.v[i];
#pragma unroll
    for (int i = 0; i < LB::NV; ++i) *reinterpret_cast<floatx4 *>(bn + i * LB::DR * T::BPITCH) = lb.v[i];
  };
  const int a_rd = TA ? (g * T::GK) * T::APITCH + wm * T::WTM + li
                      : (wm * T::WTM + li) * T::APITCH + g * T::GK;
  const int b_rd = TB ? (wn * T::WTN + li) * T::BPITCH + g * T::GK
                      : (g * T::GK) * T::BPITCH + wn * T::WTN + (PERMB ? T::FN * li : li);

  Acc acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < kRegs; ++r) acc[i][j][r] = 0.0f;

  // Scheduling-group masks (LLVM AMDGPU): matrix instructions, LDS reads, LDS
  // writes, global reads.
  constexpr int kMfma = 0x008, kDsRead = 0x100, kDsWrite = 0x200, kVmemRead = 0x020;
  // LDS read instructions per operand group: a 16-byte read per block for a
  // k-contiguous operand, scalar pairs (two per block) for an M/N-contiguous
  // one, four vector reads for the permuted B.
  constexpr int kReads = (TA ? 2 * T::FM : T::FM) + (TB ? T::FN : (PERMB ? 4 : 2 * T::FN));
  constexpr int kVecs = LA::NV + LB::NV;     // stores / loads per thread and slab

  // RAGGED (BK does not divide K): slab t >= 1 covers [t BK - ov, (t+1) BK -
  // ov), so the last slab ends at K and every load stays inside the operands,
  // and slab 0 covers [0, BK - ov): its last ov values are overwritten with
  // zeros in LDS, in both operands, so nothing is counted twice and no 0 * Inf
  // arises.  (A separate instantiation keeps the register allocation of the
  // common case untouched.)
  const int nk = RAGGED ? (p.K + BK - 1) / BK : p.K / BK;
  if constexpr (RAGGED) {
    const int ov = nk * BK - p.K;
    la.shift_k(ov);
    lb.shift_k(ov);
    la.load(ov);
    lb.load(ov);
    store(0);
    la.zero_from(As + a_st, T::APITCH, BK - ov);
    lb.zero_from(Bs + b_st, T::BPITCH, BK - ov);
  } else {
    la.load(0);
    lb.load(0);
    store(0);
  }
  __syncthreads();
  la.load(min(1, nk - 1) * BK);
  lb.load(min(1, nk - 1) * BK);
  Operands<T> o;
  read_sched_operands<MI, TA, TB, PERMB>(o, As + a_rd, Bs + b_rd, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const float *as = As + cur * T::A_STAGE + a_rd;
    const float *bs = Bs + cur * T::B_STAGE + b_rd;
#pragma unroll
    for (int q = 0; q + 1 < T::NQ; ++q) {
      Operands<T> nxt;
      read_sched_operands<MI, TA, TB, PERMB>(nxt, as, bs, q + 1);
      if (q == T::NQ / 2 - 1) {
        store(cur ^ 1);                        // slab kt+1 (a repeat at the end)
        la.load(min(kt + 2, nk - 1) * BK);     // slab kt+2, clamped
        lb.load(min(kt + 2, nk - 1) * BK);
      }
      multiply_part<T, Acc, 0, 4>(acc, o);
#pragma unroll
      for (int s = 0; s < kReads; ++s) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
      }
      if (q == T::NQ / 2 - 1) {
#pragma unroll
        for (int s = 0; s < kVecs; ++s) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kDsWrite, 1, 0);
        }
#pragma unroll
        for (int s = 0; s < kVecs; ++s) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kVmemRead, 1, 0);
        }
      }
      o = nxt;
    }
    multiply_part<T, Acc, 0, 2>(acc, o);
    __syncthreads();
    Operands<T> nxt;
    read_sched_operands<MI, TA, TB, PERMB>(nxt, As + (cur ^ 1) * T::A_STAGE + a_rd,
                                           Bs + (cur ^ 1) * T::B_STAGE + b_rd, 0);
    multiply_part<T, Acc, 2, 4>(acc, o);
#pragma unroll
    for (int s = 0; s < kReads; ++s) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
    o = nxt;
  }
  if constexpr (TAIL) {
    if (tail_t >= 0) {
      // Partial tile out in register order (value e of thread t at e*NT + t:
      // every store instruction of a wave writes 256 contiguous bytes), then
      // count this range in.  The workgroup that counts last reads every
      // partial back (its own included: the same bits), adds them in range
      // order 0, 1, ..., splits-1, resets the counter for the next call and
      // stores the tile below like a whole one.  No workgroup waits for
      // another.
      //
      // Coherence across the eight XCDs (each with its own L2) without
      // writing back or invalidating whole caches: the partials are stored
      // and loaded as agent-scope atomics (coherent at the device level, not
      // through an XCD's L2), every wave waits until its stores are
      // acknowledged before the barrier, and only then does one thread count
      // the range in with a device-scope atomic add; the last one's loads
      // come after it has seen the count.
      constexpr int NREG = T::FM * T::FN * kRegs;
      const size_t tile_part = (size_t)NREG * NT;
      float *mine = tl.part + ((size_t)tail_t * tl.splits + sidx) * tile_part + tid;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int r = 0; r < kRegs; ++r)
            __hip_atomic_store(mine + (size_t)((i * T::FN + j) * kRegs + r) * NT, acc[i][j][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      __shared__ int tail_last;
      __builtin_amdgcn_s_waitcnt(0);  // every memory operation of this wave complete
      __syncthreads();
      if (tid == 0) {
        const unsigned before =
            __hip_atomic_fetch_add(tl.flags + tail_t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tail_last = (before + 1u == (unsigned)tl.splits);
      }
      __syncthreads();
      if (!tail_last) return;
      const float *part0 = tl.part + (size_t)tail_t * tl.splits * tile_part + tid;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int r = 0; r < kRegs; ++r)
            acc[i][j][r] = __hip_atomic_load(part0 + (size_t)((i * T::FN + j) * kRegs + r) * NT, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      for (int sp = 1; sp < tl.splits; ++sp) {
        const float *ps = part0 + (size_t)sp * tile_part;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < kRegs; ++r)
              acc[i][j][r] += __hip_atomic_load(ps + (size_t)((i * T::FN + j) * kRegs + r) * NT, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      }
      if (tid == 0) __hip_atomic_store(tl.flags + tail_t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Epilogue: C = alpha*acc + beta*C for the rows and columns of this tile
  // (a shifted tile also computed some of its neighbour's).
  const int row0 = ms + wm * T::WTM;
  if constexpr (SPLITK) {
    // The partial tile goes through LDS (the operand stages are free now), a
    // chunk of RC rows at a time, so that the atomic adds of one instruction
    // cover consecutive columns of a row: each one then touches as few cache
    // lines as possible on its way to memory.
    constexpr int TP = BN + 1;                  // staged row pitch (floats)
    constexpr int FIT = (2 * T::A_STAGE) / TP;  // rows that fit in the A stages
    constexpr int RC = FIT >= BM ? BM : (FIT >= BM / 2 ? BM / 2 : BM / 4);
    static_assert(RC * TP <= 2 * T::A_STAGE && BM % RC == 0, "a chunk of rows must fit in the A stages");
#pragma unroll
    for (int c0 = 0; c0 < BM; c0 += RC) {
      __syncthreads();  // the stage (operands, or the previous chunk) is no longer read
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int r = 0; r < kRegs; ++r) {
            const int tr = wm * T::WTM + i * MI + acc_row<MI>(g, r) - c0;
            const int tc = wn * T::WTN + (PERMB ? T::FN * li + j : j * MI + li);
            if (tr >= 0 && tr < RC) As[tr * TP + tc] = acc[i][j][r];
          }
      __syncthreads();
      for (int e = tid; e < RC * BN; e += NT) {
        const int tr = e / BN, tc = e % BN;
        const int row = ms + c0 + tr, col = ns + tc;
        if (row < m0 || col < n0 || (CLAMPM && row >= p.M)) continue;
        atomicAdd(p.C + (size_t)row * (size_t)p.ldc + col, p.alpha * As[tr * TP + tc]);
      }
    }
  } else if constexpr (PERMB) {
    // FN consecutive columns per lane and row: one vector store (a group from
    // n0 on lies wholly inside the tile).  Like the slab loads, the vector
    // accesses go through copies that need only 4-byte alignment, so a leading
    // dimension or shift that is not a multiple of FN keeps them: one store per
    // column instead would touch each cache line FN times.
    const int colq = ns + wn * T::WTN + T::FN * li;
    const bool cvec = (reinterpret_cast<uintptr_t>(p.C) & 3) == 0;
    if (colq >= n0) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
          const int row = row0 + i * MI + acc_row<MI>(g, r);
          if (row < m0 || (CLAMPM && row >= p.M)) continue;
          float *c = p.C + (size_t)row * (size_t)p.ldc + colq;
          if (cvec) {
            if constexpr (T::FN == 4) {
              floatx4 v;
#pragma unroll
              for (int j = 0; j < 4; ++j) v[j] = p.alpha * acc[i][j][r];
              if (p.beta != 0.0f) {
                floatx4 old;
                __builtin_memcpy(&old, c, sizeof(old));
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = fmaf(p.beta, old[j], v[j]);
              }
              __builtin_memcpy(c, &v, sizeof(v));
            } else {
              floatx2 v;
#pragma unroll
              for (int j = 0; j < 2; ++j) v[j] = p.alpha * acc[i][j][r];
              if (p.beta != 0.0f) {
                floatx2 old;
                __builtin_memcpy(&old, c, sizeof(old));
#pragma unroll
                for (int j = 0; j < 2; ++j) v[j] = fmaf(p.beta, old[j], v[j]);
              }
              __builtin_memcpy(c, &v, sizeof(v));
            }
          } else {
#pragma unroll
            for (int j = 0; j < T::FN; ++j) store_out(c + j, acc[i][j][r], p.alpha, p.beta);
          }
        }
    } else if (colq + T::FN > n0) {
      // A group that straddles the first column of a shifted tile (only when
      // n0 - ns is not a multiple of FN): the tile's own columns only.
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
          const int row = row0 + i * MI + acc_row<MI>(g, r);
          if (row < m0 || (CLAMPM && row >= p.M)) continue;
          float *c = p.C + (size_t)row * (size_t)p.ldc + colq;
#pragma unroll
          for (int j = 0; j < T::FN; ++j)
            if (colq + j >= n0) store_out(c + j, acc[i][j][r], p.alpha, p.beta);
        }
    }
  } else {
    const int col0 = ns + wn * T::WTN + li;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int col = col0 + j * MI;
        if (col < n0) continue;
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
          const int row = row0 + i * MI + acc_row<MI>(g, r);
          if (row < m0 || (CLAMPM && row >= p.M)) continue;
          store_out(p.C + (size_t)row * (size_t)p.ldc + col, acc[i][j][r], p.alpha, p.beta);
        }
      }
  }
}

// True when sched_kernel<..., BM, BN, BK, ...> may run this problem
// (SHORTM: also with M below BM when A is not transposed).
template <int BM, int BN, int BK, bool SHORTM = false>
inline bool sched_ok(const Problem &p) {
  return p.K >= BK && (p.M >= BM || (SHORTM && !p.ta && p.M >= 1)) && p.N >= BN &&
         (reinterpret_cast<uintptr_t>(p.A) & 3) == 0 && (reinterpret_cast<uintptr_t>(p.B) & 3) == 0;
}

// Number of K ranges for a grid of `tiles` output tiles (over all batch
// slices) with two workgroups per CU: none when the tiles alone give every
// slot one, otherwise enough to, each range at least four slabs deep and a
// multiple of BK; the last range takes the rest, which is kept at least BK.
template <int BK>
static int sched_splits(long long tiles, int K, int &k_per_split) {
  const long long slots = 512;
  long long splits = (tiles >= slots) ? 1 : (slots + tiles - 1) / tiles;
  const long long max_splits = K / (4 * BK);
  if (splits > max_splits) splits = max_splits;
  k_per_split = K;
  if (splits < 2) return 1;
  long long kps = ((long long)K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  splits = ((long long)K + kps - 1) / kps;
  if (K - (splits - 1) * kps < BK) --splits;  // fold a short rest into the range before
  if (splits < 2) return 1;
  k_per_split = (int)kps;
  return (int)splits;
}

// Workspace layout of the tail form: the per-tile counters first (at most
// kTailMaxTiles of them, in kTailFlagBytes), then the partial tiles.  The
// partials of one call are capped at kTailPartBytes, which bounds the
// workspace any problem needs.
constexpr long long kTailMaxTiles = 1024;
constexpr long long kTailFlagBytes = 4096;
constexpr long long kTailPartBytes = 32LL << 20;
constexpr long long kTailWorkspaceBytes = kTailFlagBytes + kTailPartBytes;
constexpr int kTailCus = 256;  // compute units of an MI355X

// The tail plan of a grid of `tiles` output tiles (one batch slice) for a
// tile family that runs `slots` workgroups per CU: whole rounds of tiles run
// whole; the tiles of a last, partial round are each split into enough K
// ranges to fill the CUs' slots -- at most kTailMaxSplits (the workgroup
// that finishes a tile last reads every partial), each range at least four
// whole slabs, within the workspace cap.  splits == 1: no tail form (a
// whole number of rounds, or too short a K).
constexpr int kTailMaxSplits = 8;
struct TailPlan {
  int dp_tiles = 0, tail_tiles = 0, splits = 1;
  int max_range = 0;    // K depth of the deepest range
  long long bytes = 0;  // workspace needed
};
inline TailPlan tail_plan(long long tiles, int K, int slots, long long tile_floats, int BK) {
  TailPlan t;
  const long long P = (long long)kTailCus * slots;
  const long long rem = tiles % P;
  if (tiles < 1 || rem == 0 || rem > kTailMaxTiles) return t;
  long long splits = P / rem;
  const long long nkf = K / BK;
  if (splits > nkf / 4) splits = nkf / 4;
  if (splits > kTailMaxSplits) splits = kTailMaxSplits;
  const long long cap = kTailPartBytes / (rem * tile_floats * 4);
  if (splits > cap) splits = cap;
  if (splits < 2) return t;
  t.dp_tiles = (int)(tiles - rem);
  t.tail_tiles = (int)rem;
  t.splits = (int)splits;
  // slabs of the deepest range (a middle one, or the last with K's rest)
  const long long mid = (nkf + splits - 1) / splits;
  const long long last_k = K - (long long)((splits - 1) * nkf / splits) * BK;
  t.max_range = (int)(mid * BK > last_k ? mid * BK : last_k);
  t.bytes = kTailFlagBytes + rem * splits * tile_floats * 4;
  return t;
}

// Launches sched_kernel when its preconditions hold, else `fallback` (a
// variant of the same tile family that accepts every problem).  SPLIT: K may
// be split over workgroups when the tiles leave CUs idle.  SHORTM: M may be
// below BM when A is not transposed.  TAILOK: with a workspace large enough
// (and one batch slice) the last partial round of tiles takes the tail form
// (TailArgs), `slots` workgroups of this family fitting on a CU.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MINW, int BPAD,
          bool SPLIT = false, bool SHORTM = false, bool TAILOK = false, int SLOTS = 1>
static int launch_sched(const Problem &p, hipStream_t stream,
                        int (*fallback)(const Problem &, hipStream_t)) {
  if (!sched_ok<BM, BN, BK, SHORTM>(p)) return fallback(p, stream);
  const long long tiles_m = ((long long)p.M + BM - 1) / BM;
  const long long tiles_n = ((long long)p.N + BN - 1) / BN;
  if (tiles_m * tiles_n > (long long)INT_MAX) return -1;
  int k_per_split = p.K;
  const int splits = SPLIT ? sched_splits<BK>(tiles_m * tiles_n * p.batch, p.K, k_per_split) : 1;
  TailArgs tl;
  TailPlan tp;
  if constexpr (TAILOK) {
    if (p.batch == 1 && p.ws != nullptr) {
      tp = tail_plan(tiles_m * tiles_n, p.K, SLOTS, (long long)BM * BN, BK);
      if (tp.splits > 1 && (unsigned long long)tp.bytes <= p.ws_bytes) {
        tl.dp_tiles = tp.dp_tiles;
        tl.splits = tp.splits;
        tl.flags = reinterpret_cast<unsigned *>(p.ws);
        tl.part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + kTailFlagBytes);
      }
    }
  }
  const bool tail = TAILOK && tl.splits > 1;
  if (splits > 1) {
    if (splits > 65535) return -1;
    // C = beta*C first; the split workgroups then add into it.
    if (p.beta != 1.0f && launch_scale(p, stream) != 0) return -1;
  }
  // Every range but the last is a multiple of BK; the last decides.
  const bool ragged = (p.K - (splits - 1) * k_per_split) % BK != 0;
  const long long gx = tail ? (long long)tp.dp_tiles + (long long)tp.tail_tiles * tp.splits
                            : tiles_m * tiles_n;
  if (gx > (long long)INT_MAX) return -1;
  const dim3 grid((unsigned)gx, (unsigned)splits, (unsigned)p.batch);
  const dim3 block(WAVES_M * WAVES_N * 64);
  const int tm = (int)tiles_m, tn = (int)tiles_n, group_m = 8;
  // The row-clamping form only where M is below the tile (A untransposed).
  const bool short_m = SHORTM && p.M < BM;
#define SG950_SCHED_K(TA_, TB_, RG_, SK_)                                                                       \
  do {                                                                                                        \
    if constexpr (TAILOK && !(SK_)) {                                                                         \
      if (tail) {                                                                                             \
        SG950_LAUNCH((sched_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, TA_, TB_, RG_, false, false, true>), \
                     grid, block, 0, stream, p, tm, tn, group_m, k_per_split, tl);                           \
        break;                                                                                                \
      }                                                                                                       \
    }                                                                                                         \
    if constexpr (SHORTM && !(TA_)) {                                                                         \
      if (short_m) {                                                                                          \
        SG950_LAUNCH((sched_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, TA_, TB_, RG_, SK_, true>), \
                           grid, block, 0, stream, p, tm, tn, group_m, k_per_split, tl);                      \
        break;                                                                                                \
      }                                                                                                       \
    }                                                                                                         \
    SG950_LAUNCH((sched_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, MINW, BPAD, TA_, TB_, RG_, SK_>), grid,  \
                       block, 0, stream, p, tm, tn, group_m, k_per_split, tl);                                 \
  } while (0)
#define SG950_SCHED(TA_, TB_)                       \
  do {                                              \
    if (splits > 1) {                               \
      if constexpr (SPLIT) {                        \
        if (ragged)                                 \
          SG950_SCHED_K(TA_, TB_, true, true);      \
        else                                        \
          SG950_SCHED_K(TA_, TB_, false, true);     \
      }                                             \
    } else if (ragged) {                            \
      SG950_SCHED_K(TA_, TB_, true, false);         \
    } else {                                        \
      SG950_SCHED_K(TA_, TB_, false, false);        \
    }                                               \
  } while (0)
  if (!p.ta && !p.tb) {
    SG950_SCHED(false, false);
  } else if (!p.ta) {
    SG950_SCHED(false, true);
  } else if (!p.tb) {
    SG950_SCHED(true, false);
  } else {
    SG950_SCHED(true, true);
  }
#undef SG950_SCHED
#undef SG950_SCHED_K
  return 0;
}

}  // namespace sg950
