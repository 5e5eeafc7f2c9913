// sgemm_skinny.hip -- SGEMM with few rows of C (M <= 8): a matrix-vector-like
// product bound by the bandwidth of streaming B.
//
// With M <= 8 a GEMM does 2*M FLOP per element of B it reads, below the
// MI355X ridge point (about 20 FLOP/byte): the whole of B has to stream from
// HBM once, and the kernel's job is to keep enough loads in flight on every
// CU.  Three forms:
//
//   * full-K strips (moderate B): a workgroup owns 32 columns of C and runs
//     the whole K for them -- a lane loads 4 columns of 4 consecutive rows of
//     B and the matching 4 values of each row of A as 16-byte vectors, so a
//     wavefront load covers 8 rows x 128 bytes of B; each lane keeps M x 4
//     partial sums, reduced over the wave's 16 row slots by lane shuffles and
//     over the waves through LDS in a fixed order, and C = alpha*sum + beta*C
//     is written once.  One launch, no atomics, deterministic.
//   * split-K (large B, or too few column strips): the work is split over
//     columns of B (256 per workgroup: 64 lanes x a 16-byte vector, so each
//     wavefront load is 1 KiB of one row) and over K (each workgroup takes a
//     chunk of rows, its four waves a quarter of the chunk each).  A lane keeps
//     M x 4 partial sums; the four waves' sums are added through LDS in a
//     fixed order, and the workgroup adds alpha * sum into C with one float
//     atomic per element.  C is first scaled by beta in a separate launch, so
//     the result is beta*C + alpha*A*B with the K-chunks' partial sums added
//     in an unspecified order (exact on integer data; within fp32 rounding
//     otherwise).  A's values are the same for every lane and are read
//     through the scalar path.
//
//   * fixed-order split (one batch slice, with a caller's workspace): the
//     split-K grid without the atomics -- each K chunk's partial strip goes
//     to the workspace and the strip's last chunk adds them in chunk order
//     and writes C once.  One launch, deterministic; taken where K is long
//     for the columns (the full-K strips then leave CUs idle) or the columns
//     are very many.
//
// The second launch of the split form costs about 4 us on an MI355X, a fifth
// of a (1, 4096, 4096) product; the full-K form avoids it whenever the column
// strips alone give enough workgroups.
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_sched.hpp"

#include <climits>

namespace sg950 {

constexpr int kSkinnyCols = 256;  // columns of B per workgroup

// Four consecutive floats are read as one 16-byte vector through a copy,
// which needs only the 4-byte alignment of any float (as does the global
// load itself): a leading dimension that is not a multiple of 4 keeps the
// vectors.  What decides is the shape: a quad of columns of an untransposed
// B (N a multiple of 4, so the quad past the edge can be replaced by the
// last whole one), four consecutive k of a row of an untransposed A.
inline bool skinny_b_vec(const Problem &p) {
  return !p.tb && p.N % 4 == 0 && (reinterpret_cast<uintptr_t>(p.B) & 3) == 0;
}
inline bool skinny_a_vec(const Problem &p) {
  return !p.ta && (reinterpret_cast<uintptr_t>(p.A) & 3) == 0;
}
constexpr int kSkinnyWaves = 4;

// TB: B is stored N x K (op(B) = its transpose); its elements are then read
// one by one along the column (correct, not bandwidth-efficient: the table
// never picks this kernel for a transposed B).
template <int MR, bool VB, bool TB>
__global__ __launch_bounds__(kSkinnyWaves * 64) void skinny_kernel(Problem p, int kchunk) {
  select_slice(p);
  __shared__ float red[kSkinnyWaves][MR][kSkinnyCols];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = blockIdx.x * kSkinnyCols + 4 * lane;
  const int kb = blockIdx.y * kchunk;
  const int ke = min(p.K, kb + kchunk);
  const int quarter = (kchunk + kSkinnyWaves - 1) / kSkinnyWaves;
  const int k0 = min(ke, kb + w * quarter);
  const int k1 = min(ke, k0 + quarter);

  // Columns past N read the last column (in bounds, never stored).
  int cc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cc[e] = min(c0 + e, p.N - 1);
  const bool vec = VB && !TB && (c0 + 3 < p.N);
  const size_t ldb = (size_t)p.ldb;
  const size_t sa_r = p.ta ? 1 : (size_t)p.lda, sa_k = p.ta ? (size_t)p.lda : 1;

  float acc[MR][4];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;

#pragma unroll 4
  for (int k = k0; k < k1; ++k) {
    floatx4 b;
    if (TB) {
      b = floatx4{p.B[(size_t)cc[0] * ldb + k], p.B[(size_t)cc[1] * ldb + k],
                  p.B[(size_t)cc[2] * ldb + k], p.B[(size_t)cc[3] * ldb + k]};
    } else {
      const float *brow = p.B + (size_t)k * ldb;
      if (vec) {
        __builtin_memcpy(&b, brow + c0, sizeof(b));
      } else {
        b = floatx4{brow[cc[0]], brow[cc[1]], brow[cc[2]], brow[cc[3]]};
      }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (r < p.M) {
        const float a = p.A[(size_t)r * sa_r + (size_t)k * sa_k];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(a, b[e], acc[r][e]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][r][4 * lane + e] = acc[r][e];
  __syncthreads();
  if (w != 0) return;  // no barrier after this point
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (r >= p.M) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = red[0][r][4 * lane + e];
#pragma unroll
      for (int q = 1; q < kSkinnyWaves; ++q) s += red[q][r][4 * lane + e];
      if (c0 + e < p.N) atomicAdd(p.C + (size_t)r * (size_t)p.ldc + c0 + e, p.alpha * s);
    }
  }
}

constexpr int kFullKCq = 8;                  // 16-byte column quads per workgroup
constexpr int kFullKCols = 4 * kFullKCq;     // 32 columns
constexpr int kFullKWaves = 4;
constexpr int kFullKUnroll = 2;              // sweeps (4 rows each) in flight per lane
constexpr int kFullKMaxSplits = 4;           // K ranges of the split form

// Full-K strip kernel (op(B) untransposed).  Lane l takes column quad
// cq = l % 8 and row slot rr = l / 8.  In sweep i, wave w covers the 32 rows
// of B from 32(4i + w), slot rr four consecutive ones: four 16-byte loads of
// B and, per row of C, one 16-byte load of A (VA) for four k.  Columns past N
// read the last column (or quad) instead -- in bounds, never stored -- so the
// loads carry no branch and the unrolled ones issue together.  Rows of B left
// after the last whole sweep are taken one per slot, rows past K skipped.
//
// SPLIT (one batch slice, with a workspace): blockIdx.y takes the kchunk rows
// of B from blockIdx.y * kchunk, so that the strips times the ranges give
// every CU a workgroup (a strip grid of fewer workgroups than CUs leaves
// half the chip's memory requests unissued, which a cold read from HBM
// feels most); each range's partial strip goes to the workspace as
// agent-scope stores and the strip's last range adds them in range order.
template <int MR, bool VA, bool VB, bool SPLIT = false>
__global__ __launch_bounds__(kFullKWaves * 64) void skinny_fullk_kernel(Problem p, int kchunk, unsigned *flags,
                                                                         float *part) {
  select_slice(p);
  if constexpr (SPLIT) {
    const int kb = (int)blockIdx.y * kchunk;
    p.A += p.ta ? (size_t)kb * (size_t)p.lda : (size_t)kb;
    p.B += (size_t)kb * (size_t)p.ldb;
    p.K = min(p.K - kb, kchunk);
  }
  __shared__ float red[kFullKWaves][MR][kFullKCols];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cq = lane % kFullKCq, rr = lane / kFullKCq;
  const int c0 = blockIdx.x * kFullKCols + 4 * cq;
  // VB implies N % 4 == 0: quads past the edge read the last one instead.
  const int cv = min(c0, p.N - 4);
  int cc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cc[e] = min(c0 + e, p.N - 1);
  const size_t ldb = (size_t)p.ldb;
  const size_t sa_r = p.ta ? 1 : (size_t)p.lda, sa_k = p.ta ? (size_t)p.lda : 1;

  float acc[MR][4];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;

  auto load_b = [&](int k) -> floatx4 {
    const float *brow = p.B + (size_t)k * ldb;
    if constexpr (VB) {
      floatx4 v;
      __builtin_memcpy(&v, brow + cv, sizeof(v));
      return v;
    } else {
      return floatx4{brow[cc[0]], brow[cc[1]], brow[cc[2]], brow[cc[3]]};
    }
  };
  // A rows past M read row M-1 (in bounds; their sums are never stored).
  auto load_a = [&](int r, int k) -> float {
    return p.A[(size_t)min(r, p.M - 1) * sa_r + (size_t)k * sa_k];
  };
  auto load_a4 = [&](int r, int k) -> floatx4 {
    if constexpr (VA) {
      floatx4 v;
      __builtin_memcpy(&v, p.A + (size_t)min(r, p.M - 1) * sa_r + k, sizeof(v));
      return v;
    } else {
      return floatx4{load_a(r, k), load_a(r, k + 1), load_a(r, k + 2), load_a(r, k + 3)};
    }
  };

  constexpr int kSweep = kFullKWaves * 32;  // rows of B per sweep
  const int nfull = p.K / kSweep;
  int i = 0;
  for (; i + kFullKUnroll <= nfull; i += kFullKUnroll) {
    floatx4 b[kFullKUnroll][4];
    floatx4 a[kFullKUnroll][MR];
#pragma unroll
    for (int u = 0; u < kFullKUnroll; ++u) {
      const int k = (i + u) * kSweep + 32 * w + 4 * rr;
#pragma unroll
      for (int e = 0; e < 4; ++e) b[u][e] = load_b(k + e);
#pragma unroll
      for (int r = 0; r < MR; ++r) a[u][r] = load_a4(r, k);
    }
    // All loads of the batch are issued before the first use (the compiler
    // would otherwise interleave them with the FMAs and wait on each).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kFullKUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[u][r][e], b[u][e][c], acc[r][c]);
  }
  for (; i < nfull; ++i) {
    const int k = i * kSweep + 32 * w + 4 * rr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const floatx4 b = load_b(k + e);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float a = load_a(r, k + e);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a, b[c], acc[r][c]);
      }
    }
  }
  // Rows after the last whole sweep: one per slot.
  for (int k = nfull * kSweep + 8 * w + rr; k < p.K; k += kFullKWaves * 8) {
    const floatx4 b = load_b(k);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const float a = load_a(r, k);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a, b[c], acc[r][c]);
    }
  }

  // Sum over the wave's row slots (lanes cq, cq+8, ..., cq+56), then over the
  // waves in a fixed order.
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int d = kFullKCq; d < 64; d *= 2) acc[r][e] += __shfl_xor(acc[r][e], d);
  if (rr == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][r][4 * cq + e] = acc[r][e];
  }
  __syncthreads();
  if constexpr (SPLIT) {
    // Partial strip out (value r of thread t at r * 32 + t), wait until the
    // stores are acknowledged, count the range in; the last range reads the
    // partials back in range order, resets the counter and stores C.
    const int strip = blockIdx.x, sidx = blockIdx.y, splits = gridDim.y;
    constexpr int kPart = MR * kFullKCols;
    if (threadIdx.x < kFullKCols) {
      float *mine = part + ((size_t)strip * splits + sidx) * kPart + threadIdx.x;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        float s = red[0][r][threadIdx.x];
#pragma unroll
        for (int q = 1; q < kFullKWaves; ++q) s += red[q][r][threadIdx.x];
        __hip_atomic_store(mine + r * kFullKCols, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __shared__ int last_range;
    __builtin_amdgcn_s_waitcnt(0);  // every memory operation of this wave complete
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned before = __hip_atomic_fetch_add(flags + strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_range = (before + 1u == (unsigned)splits);
    }
    __syncthreads();
    if (!last_range) return;
    if (threadIdx.x < kFullKCols) {
      const int c = strip * kFullKCols + threadIdx.x;
      const float *p0 = part + (size_t)strip * splits * kPart + threadIdx.x;
      float v[kFullKMaxSplits][MR];
#pragma unroll
      for (int sp = 0; sp < kFullKMaxSplits; ++sp)
#pragma unroll
        for (int r = 0; r < MR; ++r)
          v[sp][r] = sp < splits ? __hip_atomic_load(p0 + (size_t)sp * kPart + r * kFullKCols, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0.0f;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        float s = v[0][r];
#pragma unroll
        for (int sp = 1; sp < kFullKMaxSplits; ++sp)
          if (sp < splits) s += v[sp][r];
        if (r < p.M && c < p.N) store_out(p.C + (size_t)r * (size_t)p.ldc + c, s, p.alpha, p.beta);
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(flags + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x < kFullKCols) {
    const int c = blockIdx.x * kFullKCols + threadIdx.x;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (r >= p.M || c >= p.N) continue;
      float s = red[0][r][threadIdx.x];
#pragma unroll
      for (int q = 1; q < kFullKWaves; ++q) s += red[q][r][threadIdx.x];
      store_out(p.C + (size_t)r * (size_t)p.ldc + c, s, p.alpha, p.beta);
    }
  }
}

// Fixed-order split form (one batch slice, B untransposed, a workspace).
// The grid is (column strips of 256, K chunks): each workgroup streams a
// chunk of rows of B as 1 KiB row segments (lane l: columns 4l..4l+3 of the
// strip, its wave: every fourth row of the chunk, eight rows in flight), so
// HBM sees long runs of each row instead of 128-byte pieces at a 4*N-byte
// stride.  The four waves' sums meet in LDS in a fixed order; the chunk's
// partial strip goes to the workspace as agent-scope stores (coherent across
// the XCDs), the chunk counts itself in with a device-scope atomic, and the
// chunk that counts last adds the strip's partials in chunk order and writes
// C = alpha*sum + beta*C.  One launch, no atomics on C, bitwise repeatable.
constexpr int kFixedUnroll = 8;  // rows of B in flight per wave

template <int MR, bool VB>
__global__ __launch_bounds__(kSkinnyWaves * 64) void skinny_fixed_kernel(Problem p, int kchunk,
                                                                        unsigned *flags, float *part) {
  __shared__ float red[kSkinnyWaves][MR][kSkinnyCols];
  __shared__ int last_chunk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int strip = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
  const int c0 = strip * kSkinnyCols + 4 * lane;
  const int kb = chunk * kchunk;
  const int ke = min(p.K, kb + kchunk);
  // Columns past N read the last column (VB, N a multiple of 4: the last
  // quad) -- in bounds, never stored -- so the loads carry no branch.
  const int cv = min(c0, p.N - 4);
  int cc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cc[e] = min(c0 + e, p.N - 1);
  const size_t ldb = (size_t)p.ldb;
  const size_t sa_r = p.ta ? 1 : (size_t)p.lda, sa_k = p.ta ? (size_t)p.lda : 1;
  auto load_b = [&](int k) -> floatx4 {
    const float *brow = p.B + (size_t)k * ldb;
    if constexpr (VB) {
      floatx4 v;
      __builtin_memcpy(&v, brow + cv, sizeof(v));
      return v;
    } else {
      return floatx4{brow[cc[0]], brow[cc[1]], brow[cc[2]], brow[cc[3]]};
    }
  };
  // rows of A past M read row M - 1 (their sums are never stored)
  auto load_a = [&](int r, int k) -> float { return p.A[(size_t)min(r, p.M - 1) * sa_r + (size_t)k * sa_k]; };

  float acc[MR][4];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;
  // wave w takes rows kb + w, kb + w + 4, ...
  int k = kb + w;
  for (; k + kSkinnyWaves * (kFixedUnroll - 1) < ke; k += kSkinnyWaves * kFixedUnroll) {
    floatx4 b[kFixedUnroll];
    float a[kFixedUnroll][MR];
#pragma unroll
    for (int u = 0; u < kFixedUnroll; ++u) {
      b[u] = load_b(k + kSkinnyWaves * u);
#pragma unroll
      for (int r = 0; r < MR; ++r) a[u][r] = load_a(r, k + kSkinnyWaves * u);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch issued before the first use
#pragma unroll
    for (int u = 0; u < kFixedUnroll; ++u)
#pragma unroll
      for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(a[u][r], b[u][e], acc[r][e]);
  }
  for (; k < ke; k += kSkinnyWaves) {
    const floatx4 b = load_b(k);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const float a = load_a(r, k);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(a, b[e], acc[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][r][4 * lane + e] = acc[r][e];
  __syncthreads();
  // thread t: column t of the strip, the waves' sums in order
  const size_t strip_part = (size_t)nchunks * MR * kSkinnyCols;
  float *mine = part + (size_t)strip * strip_part + (size_t)chunk * MR * kSkinnyCols + tid;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    float s = red[0][r][tid];
#pragma unroll
    for (int q = 1; q < kSkinnyWaves; ++q) s += red[q][r][tid];
    __hip_atomic_store(mine + r * kSkinnyCols, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every memory operation of this wave complete
  __syncthreads();
  if (tid == 0) {
    const unsigned before = __hip_atomic_fetch_add(flags + strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_chunk = (before + 1u == (unsigned)nchunks);
  }
  __syncthreads();
  if (!last_chunk) return;
  // The strip's last chunk: partials added in chunk order, eight chunks'
  // loads in flight at a time.
  const int col = strip * kSkinnyCols + tid;
  const float *pcol = part + (size_t)strip * strip_part + tid;
  float sum[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) sum[r] = 0.0f;
  for (int c = 0; c < nchunks; c += 8) {
    float v[8][MR];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < MR; ++r)
        v[u][r] = (c + u < nchunks) ? __hip_atomic_load(pcol + (size_t)(c + u) * MR * kSkinnyCols + r * kSkinnyCols,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < MR; ++r)
        if (c + u < nchunks) sum[r] = (c + u == 0) ? v[u][r] : sum[r] + v[u][r];
  }
  if (tid == 0) __hip_atomic_store(flags + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (col < p.N) {
#pragma unroll
    for (int r = 0; r < MR; ++r)
      if (r < p.M) store_out(p.C + (size_t)r * (size_t)p.ldc + col, sum[r], p.alpha, p.beta);
  }
}

// Chunks of the fixed-order split form: about two workgroups per CU, each
// chunk a multiple of 32 rows (the waves' batches) and at least 128.
static int skinny_fixed_kchunk(const Problem &p, long long strips) {
  long long chunks = 512 / (strips > 0 ? strips : 1);
  if (chunks < 1) chunks = 1;
  long long kc = ((long long)p.K + chunks - 1) / chunks;
  if (kc < 128) kc = 128;
  kc = (kc + 31) / 32 * 32;
  return (int)kc;
}

// Workspace bytes of the fixed-order split form for this problem (counters
// first, then the partial strips), or 0 when the form does not apply.
long long skinny_fixed_bytes(const Problem &p) {
  if (p.M < 1 || p.M > 8 || p.tb || p.batch != 1) return 0;
  const long long strips = ((long long)p.N + kSkinnyCols - 1) / kSkinnyCols;
  if (strips > kTailMaxTiles) return 0;
  const int kc = skinny_fixed_kchunk(p, strips);
  const long long chunks = ((long long)p.K + kc - 1) / kc;
  const int mr = p.M <= 1 ? 1 : (p.M <= 2 ? 2 : (p.M <= 4 ? 4 : 8));
  const long long bytes = kTailFlagBytes + strips * chunks * mr * kSkinnyCols * 4;
  return bytes <= kTailWorkspaceBytes ? bytes : 0;
}

// The fixed-order split form when it applies and the workspace holds it,
// otherwise the other few-rows forms (M <= 8).
int launch_skinny_fixed(const Problem &p, hipStream_t stream) {
  if (p.M > 8) return -1;
  const long long need = skinny_fixed_bytes(p);
  if (need == 0 || p.ws == nullptr || (unsigned long long)need > p.ws_bytes) return launch_skinny(p, stream);
  const long long strips = ((long long)p.N + kSkinnyCols - 1) / kSkinnyCols;
  const int kc = skinny_fixed_kchunk(p, strips);
  const long long chunks = ((long long)p.K + kc - 1) / kc;
  const dim3 grid((unsigned)strips, (unsigned)chunks, 1u);
  const dim3 block(kSkinnyWaves * 64);
  unsigned *flags = reinterpret_cast<unsigned *>(p.ws);
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + kTailFlagBytes);
  const bool vb = skinny_b_vec(p);
#define SG950_FIXED(MR_)                                                                                  \
  do {                                                                                                    \
    if (vb)                                                                                               \
      SG950_LAUNCH((skinny_fixed_kernel<MR_, true>), grid, block, 0, stream, p, kc, flags, part);  \
    else                                                                                                  \
      SG950_LAUNCH((skinny_fixed_kernel<MR_, false>), grid, block, 0, stream, p, kc, flags, part); \
  } while (0)
  if (p.M <= 1) {
    SG950_FIXED(1);
  } else if (p.M <= 2) {
    SG950_FIXED(2);
  } else if (p.M <= 4) {
    SG950_FIXED(4);
  } else {
    SG950_FIXED(8);
  }
#undef SG950_FIXED
  return 0;
}

// K rows per workgroup: enough workgroups (over all batch slices) for about
// four per CU, at least 64 rows (16 per wave) each, a multiple of 16.
static int skinny_kchunk(const Problem &p, long long strips) {
  const long long target = 1024;
  long long chunks = target / (strips * p.batch > 0 ? strips * p.batch : 1);
  if (chunks < 1) chunks = 1;
  long long kc = ((long long)p.K + chunks - 1) / chunks;
  if (kc < 64) kc = 64;
  kc = (kc + 15) / 16 * 16;
  return (int)kc;
}

int launch_skinny(const Problem &p, hipStream_t stream) {
  if (p.M > 8) return -1;
  // Full-K strips when the 32-column strips give at least a quarter of the
  // CUs a workgroup and B is moderate (measured: (1, 4096, 4096) 14 us
  // against 21 us for the split form with its scaling launch).
  const long long fstrips = ((long long)p.N + kFullKCols - 1) / kFullKCols;
  if (!p.tb && fstrips * p.batch >= 64 && (long long)p.N * p.K <= (1LL << 26) &&
      fstrips <= INT_MAX) {
    const dim3 fgrid((unsigned)fstrips, 1u, (unsigned)p.batch);
    const dim3 fblock(kFullKWaves * 64);
    const bool fvb = skinny_b_vec(p), fva = skinny_a_vec(p);
#define SG950_FULLK(MR_)                                                                        \
  do {                                                                                          \
    if (fva && fvb)                                                                             \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, true, true>), fgrid, fblock, 0, stream, p, p.K, nullptr, nullptr);  \
    else if (fvb)                                                                               \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, false, true>), fgrid, fblock, 0, stream, p, p.K, nullptr, nullptr); \
    else if (fva)                                                                               \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, true, false>), fgrid, fblock, 0, stream, p, p.K, nullptr, nullptr); \
    else                                                                                        \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, false, false>), fgrid, fblock, 0, stream, p, p.K, nullptr, nullptr); \
  } while (0)
    if (p.M <= 1) {
      SG950_FULLK(1);
    } else if (p.M <= 2) {
      SG950_FULLK(2);
    } else if (p.M <= 4) {
      SG950_FULLK(4);
    } else {
      SG950_FULLK(8);
    }
#undef SG950_FULLK
    return 0;
  }
  const long long strips = ((long long)p.N + kSkinnyCols - 1) / kSkinnyCols;
  const int kc = skinny_kchunk(p, strips);
  const long long chunks = ((long long)p.K + kc - 1) / kc;
  if (strips > INT_MAX || chunks > 65535) return -1;
  // C = beta*C first (zeros when beta == 0, nothing when beta == 1).
  if (p.beta != 1.0f && launch_scale(p, stream) != 0) return -1;
  const dim3 grid((unsigned)strips, (unsigned)chunks, (unsigned)p.batch);
  const dim3 block(kSkinnyWaves * 64);
  const bool vb = skinny_b_vec(p);
#define SG950_SKINNY(MR_)                                                                     \
  do {                                                                                        \
    if (p.tb)                                                                                 \
      SG950_LAUNCH((skinny_kernel<MR_, false, true>), grid, block, 0, stream, p, kc); \
    else if (vb)                                                                              \
      SG950_LAUNCH((skinny_kernel<MR_, true, false>), grid, block, 0, stream, p, kc); \
    else                                                                                      \
      SG950_LAUNCH((skinny_kernel<MR_, false, false>), grid, block, 0, stream, p, kc); \
  } while (0)
  if (p.M <= 1) {
    SG950_SKINNY(1);
  } else if (p.M <= 2) {
    SG950_SKINNY(2);
  } else if (p.M <= 4) {
    SG950_SKINNY(4);
  } else {
    SG950_SKINNY(8);
  }
#undef SG950_SKINNY
  return 0;
}

// The full-K strip kernel with K split over up to four ranges through a
// workspace (one batch slice, B untransposed), when its strips alone give
// fewer workgroups than CUs; otherwise launch_skinny.  Returns -1 for M > 8.
static int skinny_fullk_split_plan(const Problem &p, int &splits, int &kchunk, long long &bytes) {
  splits = 1;
  const long long fstrips = ((long long)p.N + kFullKCols - 1) / kFullKCols;
  if (p.M < 1 || p.M > 8 || p.tb || p.batch != 1 || fstrips < 64 || fstrips >= 256 || fstrips > 1024 ||
      (long long)p.N * p.K > (1LL << 26))
    return 0;
  constexpr int kSweep = kFullKWaves * 32;
  int want = (int)((256 + fstrips - 1) / fstrips);
  if (want > kFullKMaxSplits) want = kFullKMaxSplits;
  if (p.K < want * 4 * kSweep) return 0;  // at least four sweeps per range
  kchunk = (p.K + want - 1) / want;
  kchunk = (kchunk + kSweep - 1) / kSweep * kSweep;
  splits = (p.K + kchunk - 1) / kchunk;
  const int mr = p.M <= 1 ? 1 : (p.M <= 2 ? 2 : (p.M <= 4 ? 4 : 8));
  bytes = kTailFlagBytes + fstrips * splits * mr * kFullKCols * 4;
  return splits > 1 ? 1 : 0;
}

long long skinny_split_bytes(const Problem &p) {
  int splits = 1, kchunk = 0;
  long long bytes = 0;
  return skinny_fullk_split_plan(p, splits, kchunk, bytes) ? bytes : 0;
}

int launch_skinny_ws(const Problem &p, hipStream_t stream) {
  if (p.M > 8) return -1;
  int splits = 1, kchunk = 0;
  long long bytes = 0;
  if (!skinny_fullk_split_plan(p, splits, kchunk, bytes) || p.ws == nullptr ||
      (unsigned long long)bytes > p.ws_bytes)
    return launch_skinny(p, stream);
  const long long fstrips = ((long long)p.N + kFullKCols - 1) / kFullKCols;
  const dim3 fgrid((unsigned)fstrips, (unsigned)splits, 1u);
  const dim3 fblock(kFullKWaves * 64);
  unsigned *flags = reinterpret_cast<unsigned *>(p.ws);
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + kTailFlagBytes);
  const bool fvb = skinny_b_vec(p), fva = skinny_a_vec(p);
#define SG950_FULLKS(MR_)                                                                                \
  do {                                                                                                   \
    if (fva && fvb)                                                                                      \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, true, true, true>), fgrid, fblock, 0, stream, p, kchunk, flags, part);  \
    else if (fvb)                                                                                        \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, false, true, true>), fgrid, fblock, 0, stream, p, kchunk, flags, part); \
    else if (fva)                                                                                        \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, true, false, true>), fgrid, fblock, 0, stream, p, kchunk, flags, part); \
    else                                                                                                 \
      SG950_LAUNCH((skinny_fullk_kernel<MR_, false, false, true>), fgrid, fblock, 0, stream, p, kchunk, flags, part); \
  } while (0)
  if (p.M <= 1) {
    SG950_FULLKS(1);
  } else if (p.M <= 2) {
    SG950_FULLKS(2);
  } else if (p.M <= 4) {
    SG950_FULLKS(4);
  } else {
    SG950_FULLKS(8);
  }
#undef SG950_FULLKS
  return 0;
}

}  // namespace sg950
