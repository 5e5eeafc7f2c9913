// sgemm_fewrows.hip -- SGEMM with few rows of C (M <= 32) on the matrix
// cores: a product bound by the bandwidth of streaming B.
//
// With M <= 32 a GEMM does at most 64 FLOP per element of B it reads, near
// the MI355X ridge point, so B has to stream from HBM once with many loads in
// flight, and the arithmetic must keep up with it: the vector units cannot
// (up to 32 rows of FMAs per loaded element), the matrix cores can.
//
// A workgroup owns a strip of columns of C and all of its rows (one or two
// 16-row blocks, sharing every load of B); its eight waves take eight
// contiguous K ranges (a transposed B of 256 MiB or more: batches of K groups
// in turn, so that the waves read neighbouring bytes of each row of B
// together).  Each wave accumulates 16 x 16 blocks
// with v_mfma_f32_16x16x4f32, whose lane l supplies A[l%16][slot l/16] and
// B[slot][l%16] for the four k slots of one instruction; the k behind a slot
// is free to choose as long as A and B agree on it:
//
//   * B untransposed (k-rows): in step e of a group of 16 k the lanes of slot
//     s read row k0 + 4s + e, lane j taking CPL adjacent columns as one 4-, 8-
//     or 16-byte load (a wavefront load is four rows x 64 CPL bytes).  Value
//     c of the load feeds block c, so block c holds the columns CPL*j + c of
//     the strip (16 CPL columns); a lane's A values for the group (row l%16,
//     k0 + 4s .. 4s + 3) are one 16-byte load and serve all CPL blocks;
//   * B transposed (stored N x K): lane j of slot s reads four consecutive k
//     of each of its columns j + 16c (c < CPL), k0 + 4s .. 4s + 3, as one
//     16-byte load per column, and value e feeds instruction e of four, with
//     the matching four k of A, one A load serving all CPL column blocks.
//
// Loads of eight steps are issued before their first use (with B
// untransposed and four or more blocks per wave, one group's loads are
// issued before the previous group's matrix instructions); an untransposed
// B of 512 MiB or more, which no call finds in a cache, is read with
// non-temporal loads.  Rows past M read
// row M-1 and columns past N read column N-1 (in bounds, never stored); k
// past the end of a wave's range is skipped by selection, so a NaN or Inf
// outside the matrices cannot leak in.  The eight waves' blocks are added
// through LDS in a fixed order, each block by its own wave, and
// C = alpha*sum + beta*C is written once: one launch, no atomics,
// deterministic.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_sched.hpp"

#include <climits>

namespace sg950 {

namespace {
constexpr int kFewWaves = 8;   // waves per workgroup, each a K range
constexpr int kFewUnroll = 8;  // steps whose loads are in flight together
constexpr int kFewMaxSplits = 4;  // K chunks of the split form
}  // namespace

// NR: 16-row blocks of C (M <= 16 NR).  CPL: column blocks per lane (the
// strip is 16 CPL columns).  VB: an untransposed B's rows hold whole
// CPL-column groups (N % CPL == 0), so a lane's columns are one load.
//
// SPLIT (one batch slice, with a workspace): blockIdx.y takes the kchunk
// values of K from blockIdx.y * kchunk (the eight waves split that chunk),
// so that strips x chunks give every CU a workgroup where the strips alone
// cannot; each chunk's partial blocks go to the workspace as agent-scope
// stores and the strip's last chunk adds them in chunk order and stores C.
// W consecutive floats of B; NTL: as non-temporal loads, which do not keep
// the lines in the caches.
template <bool NTL, int W>
__device__ __forceinline__ void load_b_words(float *dst, const float *src) {
  if constexpr (NTL) {
    if constexpr (W == 4) {
      const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(src));
      dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    } else if constexpr (W == 2) {
      const floatx2 v = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(src));
      dst[0] = v[0]; dst[1] = v[1];
    } else {
      dst[0] = __builtin_nontemporal_load(src);
    }
  } else {
    __builtin_memcpy(dst, src, W * sizeof(float));
  }
}

// NTL (B untransposed): B read with non-temporal loads.  ILV (B transposed):
// the waves take batches of K groups in turn rather than one range each.
template <int NR, int CPL, bool TA, bool TB, bool VB, bool SPLIT = false, bool NTL = false, bool ILV = false>
__global__ __launch_bounds__(kFewWaves * 64) void fewrows_kernel(Problem p, int krange, int kchunk,
                                                                 unsigned *flags, float *part) {
  select_slice(p);
  if constexpr (SPLIT) {
    const int kb = (int)blockIdx.y * kchunk;
    p.A += TA ? (size_t)kb * (size_t)p.lda : (size_t)kb;
    p.B += TB ? (size_t)kb : (size_t)kb * (size_t)p.ldb;
    p.K = min(p.K - kb, kchunk);
  }
  constexpr int NB = CPL;       // 16 x 16 blocks per wave and row block
  constexpr int NC = 16 * CPL;  // columns per workgroup
  __shared__ floatx4 red[kFewWaves][NR * NB][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane % 16, sl = lane / 16;
  // Neighbouring strips share cache lines of B: give each XCD (and its L2) a
  // contiguous run of them.
  const int n0 = xcd_remap((int)blockIdx.x, (int)gridDim.x) * NC;
  int arow[NR];  // A rows of this lane, one per row block
#pragma unroll
  for (int r = 0; r < NR; ++r) arow[r] = min(16 * r + li, p.M - 1);
  const int kb = w * krange;          // this wave's K range [kb, ke)
  const int ke = min(p.K, kb + krange);
  const size_t lda = (size_t)p.lda, ldb = (size_t)p.ldb;

  floatx4 acc[NR][NB];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < NB; ++e) acc[r][e] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (!TB) {
    const int c0 = n0 + CPL * li;  // this lane's first column
    struct Cols {
      float v[CPL];
    };
    auto load_b = [&](int k) -> Cols {
      const float *row = p.B + (size_t)k * ldb;
      Cols b;
      if constexpr (VB) {
        // Whole groups: a group past N repeats the last one (never stored).
        load_b_words<NTL, CPL>(b.v, row + min(c0, p.N - CPL));
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) load_b_words<NTL, 1>(&b.v[e], row + min(c0 + e, p.N - 1));
      }
      return b;
    };
    // Four consecutive k of one of this lane's rows of op(A), for one slot.
    auto load_a4 = [&](int r, int k) -> floatx4 {
      if constexpr (!TA) {
        floatx4 v;
        __builtin_memcpy(&v, p.A + (size_t)arow[r] * lda + k, sizeof(v));
        return v;
      } else {
        const float *q = p.A + (size_t)k * lda + arow[r];
        return floatx4{q[0], q[lda], q[2 * lda], q[3 * lda]};
      }
    };
    // Groups of 16 k: slot sl takes k = k0 + 4 sl + e in step e, so a lane's
    // A values for the group are one vector.
    const int nfull = (ke > kb) ? (ke - kb) / 16 : 0;
    int t = 0;
    if constexpr (NR * CPL >= 4) {
      // Four or more blocks per wave: a group's matrix instructions take long
      // enough that the next group's loads are issued before them (two sets
      // of operand registers, the loop unrolled by two so that each set has
      // fixed registers).
      struct Group {
        Cols b[4];
        floatx4 a[NR];
      };
      auto issue = [&](Group &x, int g) {
        const int k = kb + 16 * g + 4 * sl;
#pragma unroll
        for (int r = 0; r < NR; ++r) x.a[r] = load_a4(r, k);
#pragma unroll
        for (int e = 0; e < 4; ++e) x.b[e] = load_b(k + e);
      };
      auto multiply = [&](const Group &x) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a[r][e], x.b[e].v[c], acc[r][c], 0, 0, 0);
      };
      if (nfull > 0) {
        Group x0, x1;
        issue(x0, 0);
        for (; t + 2 <= nfull; t += 2) {
          issue(x1, t + 1);
          __builtin_amdgcn_sched_barrier(0);
          multiply(x0);
          if (t + 2 < nfull) issue(x0, t + 2);
          __builtin_amdgcn_sched_barrier(0);
          multiply(x1);
        }
        if (t < nfull) multiply(x0);  // x0 holds group nfull - 1
        t = nfull;
      }
    } else {
      for (; t + kFewUnroll / 4 <= nfull; t += kFewUnroll / 4) {
        Cols b[kFewUnroll / 4][4];
        floatx4 a[kFewUnroll / 4][NR];
#pragma unroll
        for (int u = 0; u < kFewUnroll / 4; ++u) {
          const int k = kb + 16 * (t + u) + 4 * sl;
#pragma unroll
          for (int r = 0; r < NR; ++r) a[u][r] = load_a4(r, k);
#pragma unroll
          for (int e = 0; e < 4; ++e) b[u][e] = load_b(k + e);
        }
        // All loads of the batch are issued before the first use.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kFewUnroll / 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
              for (int c = 0; c < CPL; ++c)
                acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][r][e], b[u][e].v[c], acc[r][c], 0, 0, 0);
      }
    }
    for (; t < nfull; ++t) {
      const int k = kb + 16 * t + 4 * sl;
      floatx4 a[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) a[r] = load_a4(r, k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Cols b = load_b(k + e);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r][e], b.v[c], acc[r][c], 0, 0, 0);
      }
    }
    // The rest of the range (fewer than 16 k): k past ke contribute 0.
    const int kt = kb + 16 * nfull;
    if (kt < ke) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = kt + 4 * sl + e;
        const bool in = k < ke;
        const int kk = in ? k : kb;  // any in-range k; the values are replaced
        Cols b = load_b(kk);
#pragma unroll
        for (int c = 0; c < CPL; ++c) b.v[c] = in ? b.v[c] : 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float av = TA ? p.A[(size_t)kk * lda + arow[r]] : p.A[(size_t)arow[r] * lda + kk];
          const float a = in ? av : 0.0f;
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b.v[c], acc[r][c], 0, 0, 0);
        }
      }
    }
  } else {
    // Column block c of the strip: columns n0 + 16c + j; lane j reads row
    // n0 + 16c + j of the stored B (clamped to N-1).
    const float *brow[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) brow[c] = p.B + (size_t)min(n0 + 16 * c + li, p.N - 1) * ldb;
    auto load_b4 = [&](int c, int k) -> floatx4 {
      float w[4];
      load_b_words<NTL, 4>(w, brow[c] + k);
      return floatx4{w[0], w[1], w[2], w[3]};
    };
    auto load_a4 = [&](int r, int k) -> floatx4 {
      if constexpr (!TA) {
        floatx4 v;
        __builtin_memcpy(&v, p.A + (size_t)arow[r] * lda + k, sizeof(v));
        return v;
      } else {
        const float *q = p.A + (size_t)k * lda + arow[r];
        return floatx4{q[0], q[lda], q[2 * lda], q[3 * lda]};
      }
    };
    // Groups of 16 k: in group g slot sl takes k = 16g + 4sl .. + 3.  A
    // lane's A vector serves all CPL column blocks, its B vector all NR row
    // blocks.
    constexpr int UN = (kFewUnroll / (NR * CPL)) > 1 ? kFewUnroll / (NR * CPL) : 2;
    auto batch = [&](int g0) {  // groups g0 .. g0 + UN - 1, loads first
      floatx4 a[UN][NR], b[UN][CPL];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int k = 16 * (g0 + u) + 4 * sl;
#pragma unroll
        for (int r = 0; r < NR; ++r) a[u][r] = load_a4(r, k);
#pragma unroll
        for (int c = 0; c < CPL; ++c) b[u][c] = load_b4(c, k);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < UN; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][r][e], b[u][c][e], acc[r][c], 0, 0, 0);
    };
    auto one = [&](int g) {
      const int k = 16 * g + 4 * sl;
      floatx4 b[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) b[c] = load_b4(c, k);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const floatx4 a = load_a4(r, k);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[c][e], acc[r][c], 0, 0, 0);
      }
    };
    // Fewer than 16 k from kt to kend: element by element, k < kend only
    // (kt itself stands in for the k past kend, whose values are replaced).
    auto tail = [&](int kt, int kend) {
      floatx4 b[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = kt + 4 * sl + e;
          const bool in = k < kend;
          b[c][e] = in ? brow[c][in ? k : kt] : 0.0f;
        }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        floatx4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = kt + 4 * sl + e;
          const bool in = k < kend;
          const int kk = in ? k : kt;
          const float av = TA ? p.A[(size_t)kk * lda + arow[r]] : p.A[(size_t)arow[r] * lda + kk];
          a[e] = in ? av : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[c][e], acc[r][c], 0, 0, 0);
      }
    };
    if constexpr (ILV) {
      // Batches of UN groups dealt to the waves in turn, so that the eight
      // waves read neighbouring bytes of each row of B together; the groups
      // after the last whole batch and the ragged end go to the wave next
      // in turn.
      const int G = p.K / 16, nch = G / UN, rw = nch % kFewWaves;
      for (int c = w; c < nch; c += kFewWaves) batch(c * UN);
      if (w == rw) {
        for (int g = nch * UN; g < G; ++g) one(g);
        if (16 * G < p.K) tail(16 * G, p.K);
      }
    } else {
      const int g0 = kb / 16;  // (krange is a multiple of 16)
      const int nfull = (ke > kb) ? (ke - kb) / 16 : 0;
      int t = 0;
      for (; t + UN <= nfull; t += UN) batch(g0 + t);
      for (; t < nfull; ++t) one(g0 + t);
      if (kb + 16 * nfull < ke) tail(kb + 16 * nfull, ke);
    }
  }

  // Lane l holds rows 16 rb + 4*(l/16) + r of row block rb; block e's column
  // j = l%16 is column CPL*j + e of the strip (B untransposed) or 16e + j
  // (transposed).
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
#pragma unroll
    for (int e = 0; e < NB; ++e) red[w][rb * NB + e][lane] = acc[rb][e];
  __syncthreads();
  if constexpr (SPLIT) {
    // Block b's wave sum (block b by wave b mod 8, over the waves in order)
    // to the workspace: value r of lane l of block b at (b * 64 + l) * 4 + r.
    constexpr int kPart = NR * NB * 256;
    const int strip = (int)blockIdx.x, sidx = (int)blockIdx.y, splits = (int)gridDim.y;
    float *mine = part + ((size_t)strip * splits + sidx) * kPart;
    for (int blk = w; blk < NR * NB; blk += kFewWaves) {
      floatx4 s = red[0][blk][lane];
#pragma unroll
      for (int q = 1; q < kFewWaves; ++q) {
        const floatx4 v = red[q][blk][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] += v[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __hip_atomic_store(mine + (blk * 64 + lane) * 4 + r, s[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __shared__ int last_chunk;
    __builtin_amdgcn_s_waitcnt(0);  // every memory operation of this wave complete
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned before = __hip_atomic_fetch_add(flags + strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_chunk = (before + 1u == (unsigned)splits);
    }
    __syncthreads();
    if (!last_chunk) return;
    const float *p0 = part + (size_t)strip * splits * kPart;
    for (int blk = w; blk < NR * NB; blk += kFewWaves) {
      const int rb = blk / NB, e = blk % NB;
      float v[kFewMaxSplits][4];
#pragma unroll
      for (int sp = 0; sp < kFewMaxSplits; ++sp)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[sp][r] = sp < splits ? __hip_atomic_load(p0 + (size_t)sp * kPart + (blk * 64 + lane) * 4 + r,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0.0f;
      const int col = TB ? n0 + 16 * e + li : n0 + CPL * li + e;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = v[0][r];
#pragma unroll
        for (int sp = 1; sp < kFewMaxSplits; ++sp)
          if (sp < splits) s += v[sp][r];
        const int row = 16 * rb + 4 * sl + r;
        if (col < p.N && row < p.M) store_out(p.C + (size_t)row * (size_t)p.ldc + col, s, p.alpha, p.beta);
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(flags + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // Block b of the NR x NB is summed by wave b mod 8, over the waves in
  // order; no barrier after this point.
  for (int blk = w; blk < NR * NB; blk += kFewWaves) {
    const int rb = blk / NB, e = blk % NB;
    floatx4 s = red[0][blk][lane];
#pragma unroll
    for (int q = 1; q < kFewWaves; ++q) {
      const floatx4 v = red[q][blk][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += v[r];
    }
    const int col = TB ? n0 + 16 * e + li : n0 + CPL * li + e;
    if (col >= p.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rb + 4 * sl + r;
      if (row < p.M) store_out(p.C + (size_t)row * (size_t)p.ldc + col, s[r], p.alpha, p.beta);
    }
  }
}

namespace {
// (SP: the split form; kchunk, flags and part are its arguments)
struct FewSplit {
  int kchunk = 0;
  unsigned *flags = nullptr;
  float *part = nullptr;
};

template <int NR, int CPL, bool TA, bool TB, bool VB, bool SP, bool NTL = false, bool ILV = false>
void launch_fewrows_t(const Problem &p, dim3 grid, hipStream_t stream, int krange, const FewSplit &fs) {
  SG950_LAUNCH((fewrows_kernel<NR, CPL, TA, TB, VB, SP, NTL, ILV>), grid, dim3(kFewWaves * 64), 0, stream, p, krange,
               fs.kchunk, fs.flags, fs.part);
}

template <int NR, int CPL, bool TB, bool SP, bool NTL = false, bool ILV = false>
void launch_fewrows_ta(const Problem &p, dim3 grid, hipStream_t stream, int krange, bool vb, const FewSplit &fs) {
  if (p.ta) {
    if (vb)
      launch_fewrows_t<NR, CPL, true, TB, true, SP, NTL, ILV>(p, grid, stream, krange, fs);
    else
      launch_fewrows_t<NR, CPL, true, TB, false, SP, NTL, ILV>(p, grid, stream, krange, fs);
  } else {
    if (vb)
      launch_fewrows_t<NR, CPL, false, TB, true, SP, NTL, ILV>(p, grid, stream, krange, fs);
    else
      launch_fewrows_t<NR, CPL, false, TB, false, SP, NTL, ILV>(p, grid, stream, krange, fs);
  }
}

template <int NR, bool SP, bool NTL = false, bool ILV = false>
void launch_fewrows_nr(const Problem &p, dim3 grid, hipStream_t stream, int krange, int cpl, const FewSplit &fs) {
  if (p.tb) {  // (non-temporal loads only for an untransposed B)
    if (cpl == 4)
      launch_fewrows_ta<NR, 4, true, SP, false, ILV>(p, grid, stream, krange, false, fs);
    else if (cpl == 2)
      launch_fewrows_ta<NR, 2, true, SP, false, ILV>(p, grid, stream, krange, false, fs);
    else
      launch_fewrows_ta<NR, 1, true, SP, false, ILV>(p, grid, stream, krange, false, fs);
    return;
  }
  const bool vb = p.N % cpl == 0;
  if (cpl == 4)
    launch_fewrows_ta<NR, 4, false, SP, NTL>(p, grid, stream, krange, vb, fs);
  else if (cpl == 2)
    launch_fewrows_ta<NR, 2, false, SP, NTL>(p, grid, stream, krange, vb, fs);
  else
    launch_fewrows_ta<NR, 1, false, SP, NTL>(p, grid, stream, krange, vb, fs);
}
}  // namespace

// Column blocks per lane of the unsplit kernel: the most that still give the
// strips at least one workgroup per CU over the batch.
static int fewrows_cpl(const Problem &p) {
  for (int c = 4; c >= 2; c /= 2) {
    const long long strips = ((long long)p.N + 16 * c - 1) / (16 * c);
    if (strips * p.batch >= 256) return c;
  }
  return 1;
}

int fewrows_strip_cols(const Problem &p) { return 16 * fewrows_cpl(p); }

int fewrows_round_fill_pct(const Problem &p) {
  const int c = fewrows_cpl(p);
  const long long units = ((long long)p.N + 16 * c - 1) / (16 * c) * (long long)p.batch;
  if (units <= 0) return 0;
  const long long rounds = (units + 255) / 256;
  return (int)(units * 100 / (rounds * 256));
}

int launch_fewrows(const Problem &p, hipStream_t stream) {
  if (p.M < 1 || p.M > 32) return -1;
  const int cpl = fewrows_cpl(p);
  const int nc = 16 * cpl;
  const long long blocks = ((long long)p.N + nc - 1) / nc;
  if (blocks > INT_MAX) return -1;
  // Eight K ranges, each a multiple of 16 k (the groups of the four slots).
  int krange = (p.K + kFewWaves - 1) / kFewWaves;
  krange = (krange + 15) / 16 * 16;
  const dim3 grid((unsigned)blocks, 1u, (unsigned)p.batch);
  const FewSplit none;
  // An untransposed B of 512 MiB or more (twice the last-level cache) is
  // read with non-temporal loads: no call finds it in a cache anyway, and
  // streaming past the caches runs 9-14% faster ((1, 16384, 16384) 175 against
  // 192 us, (16, 16384, 8192) 88.8 against 95.9).  Below that they lose when
  // B stays cached between calls ((1, 4096, 16384) 69.9 against 49.2 us), and
  // with B transposed always (each line is read in two halves by successive
  // loads, the second of which then misses: (16, 16384, 8192) 156 against
  // 126 us).
  const long long nk = (long long)p.N * p.K * p.batch;
  const bool ntl = !p.tb && nk >= (1LL << 27);
  // A transposed B of 256 MiB or more: the waves take batches of groups in
  // turn instead of one contiguous K range each, so a workgroup's reads of
  // each row of B arrive together.  With one range per wave the reads kept
  // fewer requests in flight at a longer latency (30.5k at 2210 cycles
  // against 34.7k at 1860 for B untransposed, (16, 16384, 8192)): (16,
  // 16384, 8192) 125.6 -> 110.4 us, (1, 16384, 8192) 127 -> 102, (8, 8192,
  // 8192) cold 88 -> 62.  Smaller, it measured within a few percent either
  // way ((1, 4096, 4096) 12.1 against 12.7 us, (16, 4096, 4096) cold 20.4
  // against 19.2).
  const bool ilv = p.tb && nk >= (1LL << 26);
  if (p.M > 16) {
    if (ntl)
      launch_fewrows_nr<2, false, true>(p, grid, stream, krange, cpl, none);
    else if (ilv)
      launch_fewrows_nr<2, false, false, true>(p, grid, stream, krange, cpl, none);
    else
      launch_fewrows_nr<2, false>(p, grid, stream, krange, cpl, none);
  } else {
    if (ntl)
      launch_fewrows_nr<1, false, true>(p, grid, stream, krange, cpl, none);
    else if (ilv)
      launch_fewrows_nr<1, false, false, true>(p, grid, stream, krange, cpl, none);
    else
      launch_fewrows_nr<1, false>(p, grid, stream, krange, cpl, none);
  }
  return 0;
}

// The split form's plan: the fewest column blocks per lane (1, 2 or 4) that
// give at most 128 strips, so that at least two K chunks fit one round of
// workgroups, and as many chunks as keep strips x chunks within one
// workgroup per CU (at most four, each at least 128 values of K per wave).
// Up to 2048 columns that is one block per lane, the strips as many as they
// can be; past 8192 columns there is no plan.  (16-column strips past 2048
// columns, two chunks each, overfill the CUs and lose to the unsplit kernel:
// cold, (8, 3072, 2048) 12.5 against 11.5 us, (16, 4000, 4096) 22.1 against
// 19.5.)
static bool fewrows_split_plan(const Problem &p, int &splits, int &kchunk, long long &bytes, int &cpl) {
  splits = 1;
  cpl = 1;
  if (p.M < 1 || p.M > 32 || p.batch != 1) return false;
  long long strips = ((long long)p.N + 15) / 16;
  while (strips > 128 && cpl < 4) {
    cpl *= 2;
    strips = ((long long)p.N + 16 * cpl - 1) / (16 * cpl);
  }
  if (strips > 128) return false;
  int want = (int)(256 / strips);
  if (want > kFewMaxSplits) want = kFewMaxSplits;
  if (p.K < want * kFewWaves * 128) want = p.K / (kFewWaves * 128);
  if (want < 2) return false;
  kchunk = (p.K + want - 1) / want;
  kchunk = (kchunk + 16 * kFewWaves - 1) / (16 * kFewWaves) * (16 * kFewWaves);
  splits = (p.K + kchunk - 1) / kchunk;
  const int nr = p.M > 16 ? 2 : 1;
  bytes = kTailFlagBytes + strips * splits * nr * cpl * 256LL * 4;
  return splits > 1;
}

long long fewrows_split_bytes(const Problem &p) {
  int splits = 1, kchunk = 0, cpl = 1;
  long long bytes = 0;
  return fewrows_split_plan(p, splits, kchunk, bytes, cpl) ? bytes : 0;
}

int launch_fewrows_ws(const Problem &p, hipStream_t stream) {
  if (p.M < 1 || p.M > 32) return -1;
  int splits = 1, kchunk = 0, cpl = 1;
  long long bytes = 0;
  if (!fewrows_split_plan(p, splits, kchunk, bytes, cpl) || p.ws == nullptr ||
      (unsigned long long)bytes > p.ws_bytes)
    return launch_fewrows(p, stream);
  const long long strips = ((long long)p.N + 16 * cpl - 1) / (16 * cpl);
  int krange = (kchunk + kFewWaves - 1) / kFewWaves;
  krange = (krange + 15) / 16 * 16;
  FewSplit fs;
  fs.kchunk = kchunk;
  fs.flags = reinterpret_cast<unsigned *>(p.ws);
  fs.part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + kTailFlagBytes);
  const dim3 grid((unsigned)strips, (unsigned)splits, 1u);
  if (p.M > 16)
    launch_fewrows_nr<2, true>(p, grid, stream, krange, cpl, fs);
  else
    launch_fewrows_nr<1, true>(p, grid, stream, krange, cpl, fs);
  return 0;
}

}  // namespace sg950
