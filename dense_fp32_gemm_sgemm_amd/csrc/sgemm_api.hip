// sgemm_api.hip -- the C entry points: argument checks, variant table and the
// per-shape choice of kernel.
//
// Everything here runs on the host.  Argument errors are found before any HIP
// call; the only HIP calls are the device check (once per device), the kernel
// launch(es) and hipGetLastError.
#include "../../include/sgemm.h"
#include "sgemm_common.hpp"
#include "sgemm_launch.hpp"
#include "sgemm_sched.hpp"

#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>

namespace sg950 {
namespace {

typedef int (*Launcher)(const Problem &, hipStream_t);

// The few-rows kernel covers M <= 8; as a forced variant on a taller problem
// it runs on row blocks of 8 so that every variant accepts every problem.
int launch_skinny_any(const Problem &p, hipStream_t s) {
  for (int r = 0; r < p.M; r += 8) {
    Problem q = p;
    q.M = (p.M - r < 8) ? p.M - r : 8;
    q.A = p.ta ? p.A + r : p.A + (size_t)r * (size_t)p.lda;
    q.C = p.C + (size_t)r * (size_t)p.ldc;
    const int rc = launch_skinny(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

// The same for the fixed-order split few-rows form (which falls back to the
// few-rows kernel without a workspace).
int launch_skinny_fixed_any(const Problem &p, hipStream_t s) {
  for (int r = 0; r < p.M; r += 8) {
    Problem q = p;
    q.M = (p.M - r < 8) ? p.M - r : 8;
    q.A = p.ta ? p.A + r : p.A + (size_t)r * (size_t)p.lda;
    q.C = p.C + (size_t)r * (size_t)p.ldc;
    const int rc = launch_skinny_fixed(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

// The same for the few-rows kernel's workspace form.
int launch_skinny_ws_any(const Problem &p, hipStream_t s) {
  for (int r = 0; r < p.M; r += 8) {
    Problem q = p;
    q.M = (p.M - r < 8) ? p.M - r : 8;
    q.A = p.ta ? p.A + r : p.A + (size_t)r * (size_t)p.lda;
    q.C = p.C + (size_t)r * (size_t)p.ldc;
    const int rc = launch_skinny_ws(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

// The few-columns kernel covers N <= 16; as a forced variant on a wider
// problem it runs on column blocks of 16.
int launch_narrow_any(const Problem &p, hipStream_t s) {
  for (int c = 0; c < p.N; c += 16) {
    Problem q = p;
    q.N = (p.N - c < 16) ? p.N - c : 16;
    q.B = p.tb ? p.B + (size_t)c * (size_t)p.ldb : p.B + c;
    q.C = p.C + c;
    const int rc = launch_narrow(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

// A thin edge of C split off (defined with the automatic choice below).
int launch_edge_split(const Problem &p, hipStream_t s);

// The matrix-core few-rows kernel covers M <= 32; as a forced variant on a
// taller problem it runs on row blocks of 32.
int launch_fewrows_any(const Problem &p, hipStream_t s) {
  for (int r = 0; r < p.M; r += 32) {
    Problem q = p;
    q.M = (p.M - r < 32) ? p.M - r : 32;
    q.A = p.ta ? p.A + r : p.A + (size_t)r * (size_t)p.lda;
    q.C = p.C + (size_t)r * (size_t)p.ldc;
    const int rc = launch_fewrows(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

// The same for its workspace form.
int launch_fewrows_ws_any(const Problem &p, hipStream_t s) {
  for (int r = 0; r < p.M; r += 32) {
    Problem q = p;
    q.M = (p.M - r < 32) ? p.M - r : 32;
    q.A = p.ta ? p.A + r : p.A + (size_t)r * (size_t)p.lda;
    q.C = p.C + (size_t)r * (size_t)p.ldc;
    const int rc = launch_fewrows_ws(q, s);
    if (rc != 0) return rc;
  }
  return 0;
}

struct Variant {
  const char *name;
  Launcher launch;
};

// Stable order: tests and benchmarks address variants by index and name.
const Variant kVariants[] = {
    {"simple", launch_simple},
    {"valu_128x256x16", launch_valu_128x256},
    {"mfma32_256x256x32_4x2", launch_mfma32_256x256x32_4x2},
    {"mfma32_256x256x16_4x2", launch_mfma32_256x256x16_4x2},
    {"mfma32_128x128x32_2x2", launch_mfma32_128x128x32_2x2},
    {"mfma32_128x128x32_2x2_pipe", launch_mfma32_128x128x32_2x2_pipe},
    {"mfma32_128x128x16_2x2_w4", launch_mfma32_128x128x16_2x2_w4},
    {"mfma32_64x64x16_1x1", launch_mfma32_64x64x16_1x1},
    {"mfma16_128x128x16_2x2", launch_mfma16_128x128x16_2x2},
    {"mfma16_64x64x16_2x2", launch_mfma16_64x64x16_2x2},
    {"mfma32_128x128x32_2x2_splitk", launch_mfma32_128x128x32_2x2_splitk},
    {"mfma16_64x64x16_2x2_splitk", launch_mfma16_64x64x16_2x2_splitk},
    {"mfma32_64x64x16_1x1_splitk", launch_mfma32_64x64x16_1x1_splitk},
    {"skinny_m8", launch_skinny_any},
    {"mfma32_128x128x32_4x2", launch_mfma32_128x128x32_4x2},
    {"mfma32_128x128x64_4x2", launch_mfma32_128x128x64_4x2},
    {"mfma16_64x64x64_4x2_pipe", launch_mfma16_64x64x64_4x2_pipe},
    {"mfma32_128x128x32_4x2_splitk", launch_mfma32_128x128x32_4x2_splitk},
    {"mfma16_64x64x64_4x2_pipe_splitk", launch_mfma16_64x64x64_4x2_pipe_splitk},
    {"mfma32_256x256x32_2x2_sched", launch_mfma32_256x256x32_2x2_sched},
    {"mfma32_256x256x32_4x2_sched", launch_mfma32_256x256x32_4x2_sched},
    {"mfma32_128x128x32_4x2_sched", launch_mfma32_128x128x32_4x2_sched},
    {"mfma16_64x64x64_4x2_sched", launch_mfma16_64x64x64_4x2_sched},
    {"mfma16_128x128x64_4x2_sched", launch_mfma16_128x128x64_4x2_sched},
    {"mfma16_128x64x64_4x2_sched", launch_mfma16_128x64x64_4x2_sched},
    {"narrow_n16", launch_narrow_any},
    {"mfma16_128x128x32_2x2_sched", launch_mfma16_128x128x32_2x2_sched},
    {"fewrows_m32", launch_fewrows_any},
    {"mfma16_64x64x64_4x2_sched_splitk", launch_mfma16_64x64x64_4x2_sched_splitk},
    {"mfma16_32x64x64_2x2_sched", launch_mfma16_32x64x64_2x2_sched},
    {"mfma16_32x64x64_2x2_sched_splitk", launch_mfma16_32x64x64_2x2_sched_splitk},
    {"mfma16_128x128x32_2x2_sched_tail", launch_mfma16_128x128x32_2x2_sched_tail},
    {"mfma16_128x128x64_4x2_sched_tail", launch_mfma16_128x128x64_4x2_sched_tail},
    {"mfma16_128x64x64_4x2_sched_tail", launch_mfma16_128x64x64_4x2_sched_tail},
    {"mfma16_64x64x64_4x2_sched_tail", launch_mfma16_64x64x64_4x2_sched_tail},
    {"skinny_fixed_m8", launch_skinny_fixed_any},
    {"skinny_m8_ws", launch_skinny_ws_any},
    {"fewrows_m32_ws", launch_fewrows_ws_any},
    {"edge_split", launch_edge_split},
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

enum VariantId {
  kSimple = 0,
  kValu128 = 1,
  kMfma32_256x256x32 = 2,
  kMfma32_256x256x16 = 3,
  kMfma32_128x128x32 = 4,
  kMfma32_128x128x32_pipe = 5,
  kMfma32_128x128x16_w4 = 6,
  kMfma32_64x64x16 = 7,
  kMfma16_128x128x16 = 8,
  kMfma16_64x64x16 = 9,
  kMfma32_128x128x32_splitk = 10,
  kMfma16_64x64x16_splitk = 11,
  kMfma32_64x64x16_splitk = 12,
  kSkinny = 13,
  kMfma32_128x128x32_w8 = 14,
  kMfma32_128x128x64_w8 = 15,
  kMfma16_64x64x64_w8_pipe = 16,
  kMfma32_128x128x32_w8_splitk = 17,
  kMfma16_64x64x64_w8_pipe_splitk = 18,
  kMfma32_256x256x32_w4_sched = 19,
  kMfma32_256x256x32_w8_sched = 20,
  kMfma32_128x128x32_w8_sched = 21,
  kMfma16_64x64x64_w8_sched = 22,
  kMfma16_128x128x64_w8_sched = 23,
  kMfma16_128x64x64_w8_sched = 24,
  kNarrow = 25,
  kMfma16_128x128x32_w4_sched = 26,
  kFewRows = 27,
  kMfma16_64x64x64_w8_sched_splitk = 28,
  kMfma16_32x64x64_w4_sched = 29,
  kMfma16_32x64x64_w4_sched_splitk = 30,
  kMfma16_128x128x32_w4_sched_tail = 31,
  kMfma16_128x128x64_w8_sched_tail = 32,
  kMfma16_128x64x64_w8_sched_tail = 33,
  kMfma16_64x64x64_w8_sched_tail = 34,
  kSkinnyFixed = 35,
  kSkinnyWs = 36,
  kFewRowsWs = 37,
  kEdgeSplit = 38,
};

constexpr int kNoKernel = -100;

// Argument checks shared by every entry point (BLAS order: operations, sizes,
// then leading dimensions and strides, then pointers).  For a batch, slice z
// of A, B and C starts z*sa, z*sb, z*sc elements after the first; the slices
// of C must not overlap (those of A and B may, e.g. a shared B with sb = 0).
int check_args(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
               long long sa, const float *B, int ldb, long long sb, float beta, const float *C,
               int ldc, long long sc, int batch) {
  if ((opA != SGEMM_OP_N && opA != SGEMM_OP_T) || (opB != SGEMM_OP_N && opB != SGEMM_OP_T))
    return SGEMM_ERR_OP;
  if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_ERR_DIM;
  const int a_row = opA == SGEMM_OP_T ? M : K;  // stored row length of A
  const int b_row = opB == SGEMM_OP_T ? K : N;  // stored row length of B
  if (lda < (a_row > 1 ? a_row : 1) || ldb < (b_row > 1 ? b_row : 1) || ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_LD;
  if (sa < 0 || sb < 0 || sc < 0) return SGEMM_ERR_STRIDE;
  if (batch > 1 && M > 0 && N > 0 && sc < (long long)(M - 1) * ldc + N) return SGEMM_ERR_STRIDE;
  if (M == 0 || N == 0 || batch == 0) return SGEMM_OK;
  if (C == nullptr) return SGEMM_ERR_PTR;
  if (alpha != 0.0f && K > 0 && (A == nullptr || B == nullptr)) return SGEMM_ERR_PTR;
  (void)beta;
  return SGEMM_OK;
}

// The per-shape table.  Every entry names a variant that handles any shape,
// so the table only trades speed; the thresholds come from measured sweeps of
// every variant over the square sizes 128..8192, the rectangular shapes, one
// GPU's share of an eight-way split of 4096^3, and strided batches of small
// and mid-sized slices on an MI355X.  Work and tile counts are those of the
// whole batch.
//   * tiny problems (MNK <= 2^20) are launch-latency bound: one lane per
//     output wins;
//   * up to 32 rows of C: the B-streaming few-rows kernels (bandwidth
//     bound), on the vector units for up to four rows of a moderate B, on the
//     matrix cores otherwise;
//   * up to 16 columns of C: the A-streaming few-columns kernel;
//   * fewer than 16 rows otherwise: 64x64 tiles with K split over
//     workgroups, bound by streaming B;
//   * a short K (< 256): 256x256 tiles when they are mostly inside C and
//     fill the 256 CUs in whole rounds, then 128x128 tiles with 16-deep slabs
//     when there are as many as CUs and 90% of their area is inside C, else
//     64x64 tiles (16-deep slabs when K is not a multiple of 64);
//   * K split over workgroups on 64x64 tiles when there are fewer of them
//     than CUs and K >= 2048, unless 32-row tiles would leave fewer rows of
//     their tiles empty, M is 32 to 64 (the scored split tiles below win
//     there) or 32-row tiles took over from the few-rows kernel; when no
//     scored family's tile fits C, also with fewer 64x64 tiles than half the
//     CUs from K = 1024;
//   * otherwise the ordered slab loop on the tile family, with K split over
//     workgroups or not, with the best predicted rate -- 256x256 (four
//     waves, 128x128 wave tiles, one workgroup per CU), 128x128 (four waves,
//     32-deep slabs, two workgroups per CU), 128x128 (eight waves, 64-deep
//     slabs), 128x64, 64x64 (eight waves, two workgroups per CU) or 32x64
//     (four waves, three workgroups per CU), the last two also split: each
//     family's measured steady rate times the share of its tiles' area
//     inside C times the share of the CU time its tiles keep busy, and for a
//     split grid times the share of the rate a split of that depth keeps.  A
//     tile count just past a whole number of rounds (an odd M or N adding a
//     row or column of tiles) leaves the last round nearly empty, and smaller
//     tiles then win; so do 32-row tiles for M just past a multiple of 64.
// The ordered-loop variants fall back to their tile family's plain loop when
// the tile is larger than C or K is shorter than one slab.

// Percentage of the TM x TN tiles' area that lies inside an M x N slice.
long long tile_fill_pct(int M, int N, int TM, int TN) {
  const long long tm = ((long long)M + TM - 1) / TM, tn = ((long long)N + TN - 1) / TN;
  return (long long)M * N * 100 / (tm * TM * tn * TN);
}

constexpr long long kCus = 256;  // compute units of an MI355X

// Tile families of the ordered slab loop, for the choice among them.  Rates
// are the steady TFLOP/s of each family measured on MI355X over the shape
// sweeps with whole rounds of tiles (at K >= 2048 and at K <= 1024: the
// median of measured / (area share x busy share), device time per call from
// back-to-back graph replays, so no host launch gap inflates short calls); a shape
// gets rate x (share of the tiles' area inside C) x (share of the CU time
// the tiles keep busy).  The busiest CU holds n = ceil(tiles / 256) tiles;
// a family that fits s workgroups on a CU runs them s at a time at the
// steady rate, and a last group of j < s at `partial[j]` of it, so the CU
// takes s floor(n/s) + (n mod s) / partial[n mod s] steady tile-times.
struct TileFamily {
  int variant, bm, bn;
  double rate_long, rate_short;
  int slots;
  double partial[3];  // [j]: rate with j < slots workgroups on the CU
  bool short_m;       // also runs M < bm (A untransposed)
};
constexpr TileFamily kTileFamilies[] = {
    {kMfma32_256x256x32_w4_sched, 256, 256, 147.5, 141.0, 1, {0.0, 0.0, 0.0}, false},
    {kMfma16_128x128x32_w4_sched, 128, 128, 146.5, 140.0, 2, {0.0, 0.95, 0.0}, false},
    {kMfma16_128x128x64_w8_sched, 128, 128, 141.0, 131.5, 1, {0.0, 0.0, 0.0}, false},
    {kMfma16_128x64x64_w8_sched, 128, 64, 135.0, 122.5, 1, {0.0, 0.0, 0.0}, false},
    {kMfma16_64x64x64_w8_sched, 64, 64, 132.5, 123.5, 2, {0.0, 0.92, 0.0}, false},
    {kMfma16_32x64x64_w4_sched, 32, 64, 124.0, 112.5, 3, {0.0, 0.75, 0.93}, true},
};
// The same loops with K split over workgroups (atomics after a beta-scaling
// launch), priced by the unsplit family's rate at the range depth.
struct SplitFamily {
  int variant;
  TileFamily base;
};
constexpr SplitFamily kSplitFamilies[] = {
    {kMfma16_64x64x64_w8_sched_splitk, kTileFamilies[4]},
    {kMfma16_32x64x64_w4_sched_splitk, kTileFamilies[5]},
};
// Share of the unsplit rate kept by a split grid whose ranges are k deep
// (fitted to split-K runs on MI355X: 0.94-0.98 at k = 4096, 0.92-0.93 at
// 2048, 0.76 at 1024, 0.59 at 512; the atomic adds of the tile and the
// shorter pipeline both weigh more as the range shrinks).
double split_efficiency(double k) {
  const double r = 4096.0 / k;
  // Floored at one half below the measured depths (0.59 at k = 512): a grid
  // of a few dozen workgroups is slower than any split of it.
  return fmax(0.5, 1.0 / (1.0 + 0.02 * r * r));
}

// Steady rate of a family for k-deep work per tile (linear between k = 1024
// and 2048).
double family_rate_full(const TileFamily &f, double k) {
  if (k >= 2048.0) return f.rate_long;
  if (k <= 1024.0) return f.rate_short;
  return f.rate_short + (f.rate_long - f.rate_short) * (k - 1024.0) / 1024.0;
}

long long family_tiles(const TileFamily &f, const Problem &p) {
  return ((long long)p.M + f.bm - 1) / f.bm * (((long long)p.N + f.bn - 1) / f.bn) * (long long)p.batch;
}

// Share of the family's tile area that lies inside C.
double family_fill(const TileFamily &f, const Problem &p) {
  const long long tm = ((long long)p.M + f.bm - 1) / f.bm, tn = ((long long)p.N + f.bn - 1) / f.bn;
  return (double)p.M * (double)p.N / ((double)(tm * f.bm) * (double)(tn * f.bn));
}

// Share of the CU time that `units` workgroups of a family keep busy.
double round_fill(const TileFamily &f, long long units) {
  const long long n = (units + kCus - 1) / kCus;  // on the busiest CU
  const long long rest = n % f.slots;
  const double span = (double)(n - rest) + (rest ? (double)rest / f.partial[rest] : 0.0);
  return (double)units / ((double)kCus * span);
}

// The ordered loop's own preconditions on the shape (else it runs the plain
// fallback loop, which the rates do not describe).
bool family_fits(const TileFamily &f, const Problem &p) {
  return (p.M >= f.bm || (f.short_m && !p.ta)) && p.N >= f.bn;
}

// Predicted rate of a family on this problem: steady rate x area fill x
// round fill.
double family_rate(const TileFamily &f, const Problem &p) {
  return family_rate_full(f, (double)p.K) * family_fill(f, p) * round_fill(f, family_tiles(f, p));
}

// Predicted rate of a split family (0 when it would not split): the unsplit
// rate at the range depth x the split efficiency x area fill x round fill of
// tiles x ranges.
double split_rate(const SplitFamily &sf, const Problem &p) {
  const long long tiles = family_tiles(sf.base, p);
  int kps = p.K;
  const int splits = sched_splits<64>(tiles, p.K, kps);
  if (splits < 2) return 0.0;
  const double k = (double)p.K / splits;
  return family_rate_full(sf.base, k) * split_efficiency(k) * family_fill(sf.base, p) *
         round_fill(sf.base, tiles * splits);
}

// The same loops with the fixed-order split of the last partial round of
// tiles (workspace entry points only): whole rounds at the family's steady
// rate, and the last round's tiles split into K ranges that fill the slots,
// each range at the rate a split of that depth keeps.
// (whole_round: taken only after at least one whole round of tiles -- the
// 64x64 tail form never beat the other choices on a grid of a single,
// partial round, where its predicted rate ran 5-30% high.)
struct TailFamily {
  int variant;
  TileFamily base;
  int bk;
  bool whole_round;
};
constexpr TailFamily kTailFamilies[] = {
    {kMfma16_128x128x32_w4_sched_tail, kTileFamilies[1], 32, false},
    {kMfma16_128x128x64_w8_sched_tail, kTileFamilies[2], 64, false},
    {kMfma16_128x64x64_w8_sched_tail, kTileFamilies[3], 64, false},
    {kMfma16_64x64x64_w8_sched_tail, kTileFamilies[4], 64, true},
};

// Share of the rate a tail range of depth k (K values) keeps when its tile
// was split `splits` ways: the range's own slabs against those plus a fixed
// cost (its pipeline's start, about 120 values of k) and the partial tiles
// written and read back (about 20 per split).  Least-squares fit (in log
// rate) to the 195 tail-form timings of the tile-choice table on MI355X
// (device time per call); e.g. 0.45 for 191-deep ranges of 128x128 tiles in
// seven ((4095, 4097, 1023)), 0.80 for 768-deep ranges in four (3000^3).
double tail_efficiency(double k, int splits) { return k / (k + 120.0 + 20.0 * splits); }

TailPlan family_tail_plan(const TailFamily &tf, const Problem &p) {
  return tail_plan(family_tiles(tf.base, p), p.K, tf.base.slots, (long long)tf.base.bm * tf.base.bn, tf.bk);
}

// Predicted rate of a tail family (0 when it would not take the tail form:
// a batch, no room in the workspace, whole rounds, too short a K).  In
// steady tile-times on the busiest CU: the whole rounds' tiles, then the
// last round's ranges there (each k_per_split/K of a tile, at the split
// efficiency of its depth, and at the lone-workgroup rate when fewer than
// the family's slots share the CU).
double tail_rate(const TailFamily &tf, const Problem &p) {
  if (p.batch != 1 || p.ws == nullptr) return 0.0;
  const TailPlan tp = family_tail_plan(tf, p);
  if (tp.splits < 2 || (unsigned long long)tp.bytes > p.ws_bytes) return 0.0;
  if (tf.whole_round && tp.dp_tiles == 0) return 0.0;
  const TileFamily &f = tf.base;
  const long long tiles = family_tiles(f, p);
  const double whole = (double)tp.dp_tiles / (double)kCus;  // tiles per CU in whole rounds
  const long long wgs = (long long)tp.tail_tiles * tp.splits;
  const long long per_cu = (wgs + kCus - 1) / kCus;
  const double frac = (double)tp.max_range / (double)p.K;
  double last = (double)per_cu * frac / tail_efficiency((double)tp.max_range, tp.splits);
  if (per_cu < f.slots) last /= f.partial[per_cu];
  const double span = whole + last;
  return family_rate_full(f, (double)p.K) * family_fill(f, p) * (double)tiles / ((double)kCus * span);
}

// Process-wide atomics mode (sgemm_set_atomics_mode).
std::atomic<int> g_atomics_mode{SGEMM_ATOMICS_ALLOWED};

// True when the vector-unit few-rows kernel takes its full-K form (one pass,
// fixed-order sums) rather than its split form (atomics).
bool skinny_full_k(const Problem &p) {
  return !p.tb && ((long long)p.N + 31) / 32 * p.batch >= 64 && (long long)p.N * p.K <= (1LL << 26);
}

// Edge split: a dimension of C that overruns a family's tiles by a thin edge
// (1 to 32 rows or columns) costs that family a whole extra row or column
// of tiles -- at (4095, 4097, 1023) the 256x256 tiles number 16 x 17, one
// round of 256 and a second of 16 one-column tiles.  Splitting the edge off
// leaves the bulk to the tiles (whole rounds) and gives the thin strip to
// the few-columns or few-rows kernel, one launch after the other on the
// stream.  side 0: columns (keep = the bulk's N), 1: rows (keep = its M).
struct EdgePlan {
  int side = -1;
  int keep = 0;
  double rate = 0.0;  // predicted TFLOP/s of the two launches together
};

// The bulk (thin = false) or the thin strip of C and the operands it reads.
Problem edge_part(const Problem &p, int side, int keep, bool thin) {
  Problem q = p;
  if (side == 0) {
    if (!thin) {
      q.N = keep;
    } else {
      q.N = p.N - keep;
      q.C = p.C + keep;
      q.B = p.tb ? p.B + (size_t)keep * (size_t)p.ldb : p.B + keep;
    }
  } else {
    if (!thin) {
      q.M = keep;
    } else {
      q.M = p.M - keep;
      q.C = p.C + (size_t)keep * (size_t)p.ldc;
      q.A = p.ta ? p.A + keep : p.A + (size_t)keep * (size_t)p.lda;
    }
  }
  return q;
}

// The thin strip as launches: a column edge wider than the few-columns
// kernel's 16 goes as two strips (16 columns, then the rest).  Returns how
// many of out[] it filled.
int thin_parts(const Problem &p, int side, int keep, Problem (&out)[2]) {
  out[0] = edge_part(p, side, keep, true);
  if (side != 0 || out[0].N <= 16) return 1;
  out[1] = edge_part(p, side, keep + 16, true);
  out[0].N = 16;
  return 2;
}

// Microseconds a thin strip takes: a launch and a stream over its operands at
// 4 TB/s, slower when its long side is short of 4096 (the few-columns and
// few-rows kernels spread over that side).  Measured (us, alone, warm):
// (4095, 1, 1023) 6.5 (model 7.2), (8191, 1, 8191) 55 (70), (512, 1, 4096)
// 12.0 (19.8), (2047, 1, 4095) 14.9 (19.8), (1, 8192, 1024) 5.8 (11.4).
double thin_us(const Problem &t) {
  const double bytes = 4.0 * ((double)t.M * t.K + (double)t.K * t.N + (double)t.M * t.N) * (double)t.batch;
  const double side = (double)(t.M > t.N ? t.M : t.N) * (double)t.batch;
  return 3.0 + bytes / (4.0e6 * fmin(1.0, side / 4096.0));
}

// depth 1: the bulk may itself split its other edge off (both dimensions
// thin, as at (4097, 4097, 4097)); it then goes through the automatic choice
// again, which takes that second split by the same prediction.
EdgePlan edge_plan(const Problem &p, int depth = 1) {
  EdgePlan best;
  // (the family rates are fitted from a K of about 1024 up: at (1023, 8193,
  // 257) the split ran 64 against 75 TFLOP/s on whole 64x64 tiles)
  if (p.K < 1000) return best;
  const double flops = 2.0 * (double)p.M * p.N * p.K * (double)p.batch;
  for (const TileFamily &f : kTileFamilies) {
    for (int side = 0; side < 2; ++side) {
      const int dim = side == 0 ? p.N : p.M, tile = side == 0 ? f.bn : f.bm;
      const int r = dim % tile;
      // (edges of up to 32: the few-rows kernels take 32 rows, the
      // few-columns kernel 16 columns a launch)
      if (r < 1 || r > 32 || dim <= tile) continue;
      const Problem bulk = edge_part(p, side, dim - r, false);
      if (!family_fits(f, bulk)) continue;
      double rb = family_rate(f, bulk);
      if (depth > 0) rb = fmax(rb, edge_plan(bulk, depth - 1).rate);
      if (rb <= 0.0) continue;
      Problem parts[2];
      const int np = thin_parts(p, side, dim - r, parts);
      double t = 2.0 * (double)bulk.M * bulk.N * bulk.K * (double)bulk.batch / (rb * 1e6);
      for (int i = 0; i < np; ++i) t += thin_us(parts[i]);
      const double rate = flops / (t * 1e6);
      if (rate > best.rate) {
        best.side = side;
        best.keep = dim - r;
        best.rate = rate;
      }
    }
  }
  return best;
}

// The automatic choice.  atomics: whether variants that add partial sums into
// C with atomics (an order the hardware decides) may be taken.
int choose_variant(const Problem &p, bool atomics) {
  const long long batch = p.batch;
  const long long work = (long long)p.M * p.N * p.K * batch;
  const long long nk = (long long)p.N * p.K * batch;
  // Few rows and enough of B: bound by streaming B.  The vector-unit kernel
  // for up to four rows of a moderate B read in full-K strips, the matrix-core
  // kernel for up to 32 rows when its column strips fill the CUs (with a
  // transposed B, above 16 rows only for wide strips or a K up to 4096).
  // 17 to 32 rows with a large B go to 32-row tiles instead (split over K
  // when they are few; below 32 rows only with A untransposed, the tile then
  // reading row M - 1 for the rows past M), which stream B as well with better
  // matrix-core use ((32, 8192, 8192): 48.6 against 60.7 us, (32, 4096,
  // 16384) 55.8 against 82.3); below N*K = 2^25 the few-rows kernel stays
  // ahead.  With B transposed the tiles win from N*K = 2^22 when K is at
  // least N (above 16 rows) or twice N (9 to 16 rows): (24, 4096, 4096) 20.9
  // against 23.5 us, (16, 4096, 16384) 48.4 against 63.9; with N above K
  // (above K/2) the few-rows kernel wins.
  const bool tb_long_k = p.tb && (p.M > 16 ? p.K >= p.N : (p.M > 8 && p.K >= 2LL * p.N));
  const bool rows32_fits = p.N >= 64 && (p.M == 32 || (!p.ta && p.M > 8 && p.M < 32));
  const bool rows32_tiles =
      atomics && rows32_fits &&
      ((nk >= (1LL << 25) && p.M > 16) || (nk >= (1LL << 22) && tb_long_k));
  if (p.M <= 32 && p.N >= 64 && nk >= (1LL << 20) && !rows32_tiles) {
    const long long nb = (long long)p.N * batch;  // columns over the batch
    const bool valu_ok = !p.tb && p.M <= 8;
    // With a workspace, up to four rows and a full-K strip grid of fewer
    // workgroups than CUs, the vector-unit kernel's strips split over K
    // (`skinny_m8_ws`), which fills the CUs' memory queues: cold (1, 4096,
    // 4096) 15.1 against 19.5 us, (1, 2048, 8192) 15.8 against 34.5.
    const long long split_need = skinny_split_bytes(p);
    const bool ws_split = valu_ok && p.M <= 4 && batch == 1 && p.ws != nullptr && split_need > 0 &&
                          (unsigned long long)split_need <= p.ws_bytes;
    // Otherwise, with a workspace that holds it, the matrix-core few-rows
    // kernel split over K (`fewrows_m32_ws`, up to 2048 columns): up to 16
    // rows from 64 strips of 16 columns (1009 columns) at a K up to 32768
    // (as far as measured), or from fewer at a K up to 4096 (with fewer
    // strips than 64 a longer K fills too few CUs); above 16 rows where the
    // unsplit kernel is chosen below.
    // Cold, operands rotated past the last-level cache: (8, 1024, 8192)
    // 13.7 us against 31.3 on the fixed-order vector-unit form, (16, 1024,
    // 8192) 15.0 against 39.9 unsplit, (4, 1024, 4096) with B transposed 8.1
    // against 11.1 on split 64x64 tiles.
    const long long few_need = fewrows_split_bytes(p);
    const bool few_fits = p.ws != nullptr && few_need > 0 && (unsigned long long)few_need <= p.ws_bytes;
    const bool few_ws = !ws_split && p.N <= 2048 && few_fits;
    if (few_ws && p.M <= 16 && p.K <= (p.N > 1008 ? 32768 : 4096)) return kFewRowsWs;
    // Past 2048 columns (wider strips, at most 128 of them), with B
    // untransposed and K at least 4096, where the unsplit kernel's grid
    // fills less than 80% of its last round of workgroups (3072 columns: 192
    // strips, 6144: 384) -- ahead of the vector-unit strips split over K as
    // well -- or, above four rows, where its strips are 16 columns wide (up
    // to about 8192 columns: each row of B read in half lines); up to eight
    // rows only while N*K <= 2^26 (beyond it the fixed-order vector-unit
    // split streams B better: (4, 6144, 16384) 69 us against 78).  Cold:
    // (16, 6144, 4096) 25.4 against 46.6 us unsplit, (16, 3072, 8192) 31.3
    // against 45.0, (1, 3072, 8192) 25.0 against 29.9 on the vector-unit
    // split, (8, 6144, 8192) 42.8 against 78.9, (16, 4096, 16384) 64.8
    // against 85.3, (24, 4096, 4096) 23.2 against 28.4; at four rows or
    // fewer and 4096 columns the vector-unit split stays ahead ((4, 4096,
    // 4096) 16.5 against 19.8).  (With B transposed the unsplit kernel keeps
    // up: the split ran slower cold.)
    if (few_fits && !p.tb && p.N > 2048 && p.K >= 4096 && (p.M > 8 || (long long)p.N * p.K <= (1LL << 26)) &&
        (fewrows_round_fill_pct(p) < 80 || (p.M > 4 && fewrows_strip_cols(p) == 16)))
      return kFewRowsWs;
    // A K of 16N or more: too few columns for the streaming kernels' strips
    // and a long K each; split-K 64x64 tiles spread it over the CUs
    // ((1, 1024, 16384) 23.2 us against 36.2 on the vector-unit kernel's
    // split form, (8, 1024, 16384) 23.9 against 45.9) -- except at four rows
    // or fewer with K above 16384, where the fixed-order split (with a
    // workspace: (1, 1024, 65536) 53 against 78.5 us cold) or, for 2048
    // columns and more and K from 65536, the vector-unit kernel's split form
    // ((1, 2048, 65536) 101 against 151) stream B better.
    if (valu_ok && atomics && batch == 1 && p.K >= 16LL * p.N) {
      const long long need = skinny_fixed_bytes(p);
      const bool fixed_better = p.ws != nullptr && p.M <= 4 && p.K > 16384 && need > 0 &&
                                (unsigned long long)need <= p.ws_bytes;
      if (!fixed_better) {
        if (p.M <= 4 && p.N >= 2048 && p.K >= 65536) return kSkinny;
        return kMfma16_64x64x64_w8_pipe_splitk;
      }
    }
    // With a workspace that holds it: the fixed-order split few-rows form
    // where K is long for the columns (at least 2N, and N*K from 2^21 at one
    // or two rows, 2^22 up to four, 2^23 up to eight with K <= 16384), or
    // the columns very many and K short -- measured cold (operands rotated
    // past the last-level cache): (1, 2048, 16384) 33 against 63 us,
    // (1, 1024, 4096) 9.9 against 16, (8, 4096, 16384) 62 against 75,
    // (1, 65536, 2048) 86.5 against 103; the strips split over K where
    // `ws_split` holds.
    if (valu_ok && batch == 1 && p.ws != nullptr) {
      const long long need = skinny_fixed_bytes(p);
      const long long min_nk = p.M <= 2 ? (1LL << 21) : (p.M <= 4 ? (1LL << 22) : (1LL << 23));
      const bool long_k = p.K >= 2LL * p.N && nk >= min_nk && (p.M <= 4 || p.K <= 16384);
      if (need > 0 && (unsigned long long)need <= p.ws_bytes && (long_k || (p.N >= 32768 && p.K <= 2048)))
        return ws_split ? kSkinnyWs : kSkinnyFixed;
    }
    if (valu_ok && p.M <= 4 && p.N >= 2048 && p.K >= 2048 && (long long)p.N * p.K <= (1LL << 26) &&
        (p.M <= 2 || p.N >= 4096))
      return ws_split ? kSkinnyWs : kSkinny;
    // (B transposed, up to 16 rows: from 1024 columns at a K up to 2048,
    // (8, 1024, 1024) 4.8 against 8.8 us on split 64x64 tiles.)
    const bool fewrows =
        p.tb ? (p.M <= 16 ? (nb >= 2048 || (batch == 1 && p.N >= 1024 && p.K <= 2048))
                          : (nb >= 8192 || (nb >= 2048 && p.K <= 4096)))
             : nb >= (p.M <= 16 ? 1024 : 2048);
    if (fewrows) return few_ws ? kFewRowsWs : kFewRows;
    if (valu_ok && (atomics || skinny_full_k(p))) return ws_split ? kSkinnyWs : kSkinny;
  }
  // 64x64 tiles with 16-deep slabs, split over K when atomics are allowed.
  const int m16 = atomics ? kMfma16_64x64x16_splitk : kMfma16_64x64x16;
  // (the one-lane kernel reads a transposed B with a stride: small tiles then)
  if (work <= (1LL << 20)) return p.tb ? m16 : kSimple;
  // Few columns: the A-streaming few-columns kernel.
  if (p.N <= 16 && p.M >= 16) return kNarrow;
  // Few rows: bound by streaming B; 64x64 tiles with K split over workgroups
  // (16-deep slabs for a short ragged K).
  if (!rows32_tiles && (p.M < 16 || p.N < 16))
    return (p.K < 256 && p.K % 64 != 0)
               ? m16
               : (atomics ? kMfma16_64x64x64_w8_pipe_splitk : kMfma16_64x64x64_w8_pipe);
  const long long t256 = ((long long)p.M + 255) / 256 * (((long long)p.N + 255) / 256) * batch;
  const long long t128 = ((long long)p.M + 127) / 128 * (((long long)p.N + 127) / 128) * batch;
  const long long t64 = ((long long)p.M + 63) / 64 * (((long long)p.N + 63) / 64) * batch;
  const long long cus = kCus;
  // A short K: wide tiles with 16-deep slabs when they fill the CUs twice
  // (256x256 once), else 64x64 tiles (16-deep slabs when K is not a multiple
  // of 64, since a 64-deep slab would be mostly padding), or 32x64 tiles
  // while the 64x64 ones are fewer than the CUs (device time: (512, 512,
  // 128) 3.65 against 4.61 us, (128, 4096, 128) 3.84 against 4.78, 32
  // slices of 96^3 4.06 against 5.2 on 16-deep 64x64 tiles; (2048, 2048,
  // 128) 14.5 on 64x64 tiles against 16.4 on 128x128).
  if (p.K < 256) {
    if (t256 >= cus && tile_fill_pct(p.M, p.N, 256, 256) >= 75) {
      const long long tail = t256 % cus;
      if (tail == 0 || tail * 100 >= cus * 85 || t256 >= 4 * cus) return kMfma32_256x256x32_w4_sched;
    }
    if (t128 >= 2 * cus && tile_fill_pct(p.M, p.N, 128, 128) >= 90) return kMfma32_128x128x16_w4;
    if (t64 < cus && p.K >= 64 && p.N >= 64 && (p.M >= 32 || !p.ta)) return kMfma16_32x64x64_w4_sched;
    return (p.K % 64 != 0) ? m16 : kMfma16_64x64x64_w8_sched;
  }
  // Too few tiles for the CUs and a long K: split K over workgroups on 64x64
  // tiles, unless 32-row tiles leave fewer rows empty or took over from the
  // few-rows kernel above (then the scores below weigh both).
  const bool rows32_fill_better =
      p.M >= 32 && p.N >= 64 && tile_fill_pct(p.M, p.N, 32, 64) > tile_fill_pct(p.M, p.N, 64, 64);
  // (32 to 64 rows: the ordered loop's split tiles, scored below, beat it by
  // 3-8%: (48, 8192, 8192) 80.7 against 78.5, (64, 8192, 8192) 111.5 against
  // 102.9 TFLOP/s.)
  const bool split_tiles_fit = p.M >= 32 && p.M <= 64 && p.N >= 64;
  // (A K below 2048 is left to the scores as well: (300, 1000, 1024) 21.3 us
  // here against 15.4 on unsplit 32x64 tiles, (128, 1024, 1024) 15.0 against
  // 12.9 on split ones.)
  if (atomics && !rows32_fill_better && !rows32_tiles && !split_tiles_fit && t64 < cus && p.K >= 2048)
    return kMfma16_64x64x64_w8_pipe_splitk;
  // Otherwise the ordered-loop tile family, split or not, with the best
  // predicted rate.
  int best = kMfma16_64x64x64_w8_sched;
  double best_rate = -1.0;
  for (const TileFamily &f : kTileFamilies) {
    if (!family_fits(f, p)) continue;
    const double r = family_rate(f, p);
    if (r > best_rate) best_rate = r, best = f.variant;
  }
  for (const SplitFamily &sf : kSplitFamilies) {
    if (!atomics || !family_fits(sf.base, p)) continue;
    const double r = split_rate(sf, p);
    if (r > best_rate) best_rate = r, best = sf.variant;
  }
  // With a workspace: the fixed-order tail forms (no atomics on C).
  for (const TailFamily &tf : kTailFamilies) {
    if (!family_fits(tf.base, p)) continue;
    const double r = tail_rate(tf, p);
    if (r > best_rate) best_rate = r, best = tf.variant;
  }
  // A thin edge split off, where that is predicted faster by 3% or more.
  const EdgePlan ep = edge_plan(p);
  if (ep.side >= 0 && ep.rate > 1.03 * best_rate) return kEdgeSplit;
  // No family's tile fits C (fewer than 32 rows with A transposed, or fewer
  // than 64 columns): few tiles with a long K still split K over workgroups.
  if (best_rate < 0.0 && atomics && ((t64 < cus / 2 && p.K >= 1024) || (t64 < cus && p.K >= 2048)))
    return kMfma16_64x64x64_w8_pipe_splitk;
  return best;
}

// The edge split: the bulk and the thin strip, each through the automatic
// choice, one after the other on the stream.  Without a thin edge (as a
// forced variant) the whole problem goes through the automatic choice.
int launch_edge_split(const Problem &p, hipStream_t s) {
  const bool atomics = g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED;
  const EdgePlan ep = edge_plan(p);
  if (ep.side < 0) return kVariants[choose_variant(p, atomics)].launch(p, s);
  const Problem bulk = edge_part(p, ep.side, ep.keep, false);
  if (kVariants[choose_variant(bulk, atomics)].launch(bulk, s) != 0) return -1;
  Problem parts[2];
  const int np = thin_parts(p, ep.side, ep.keep, parts);
  for (int i = 0; i < np; ++i)
    if (kVariants[choose_variant(parts[i], atomics)].launch(parts[i], s) != 0) return -1;
  return 0;
}

std::atomic<int> g_device_ok[64];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SGEMM_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return SGEMM_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SGEMM_ERR_DEVICE;
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? SGEMM_OK : SGEMM_ERR_DEVICE;
}

constexpr int kMaxGridZ = 65535;

// Enqueues (or, with the launch plan set dry, only checks) every launch of
// one call: grids hold at most 65535 batch slices, so larger batches go in
// chunks.  Returns 0, or -1 when some launch cannot be made.
int launch_all(const Problem &p, int v, bool no_product, hipStream_t s) {
  for (int z0 = 0; z0 < p.batch; z0 += kMaxGridZ) {
    Problem q = p;
    q.batch = (p.batch - z0 < kMaxGridZ) ? p.batch - z0 : kMaxGridZ;
    q.A = p.A ? p.A + (size_t)z0 * (size_t)p.sa : nullptr;
    q.B = p.B ? p.B + (size_t)z0 * (size_t)p.sb : nullptr;
    q.C = p.C + (size_t)z0 * (size_t)p.sc;
    const int rc = no_product ? launch_scale(q, s) : kVariants[v].launch(q, s);
    if (rc != 0) return -1;
  }
  return 0;
}

// The launch plan of a call: every launch of every chunk checked against the
// grid limits with nothing enqueued.  True when all of them fit.
bool plan_fits(const Problem &p, int v, bool no_product) {
  LaunchPlan &lp = launch_plan();
  lp.dry = true;
  lp.failed = false;
  const int rc = launch_all(p, v, no_product, nullptr);
  const bool ok = rc == 0 && !lp.failed;
  lp.dry = false;
  lp.failed = false;
  return ok;
}

// Workspaces must be 16-byte aligned.
bool ws_aligned(const void *ws) { return (reinterpret_cast<uintptr_t>(ws) & 15) == 0; }

int run(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, long long sa,
        const float *B, int ldb, long long sb, float beta, float *C, int ldc, long long sc,
        int batch, void *ws, unsigned long long ws_bytes, void *stream, int variant) {
  int st = check_args(opA, opB, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch);
  if (st != SGEMM_OK) return st;
  if (variant < -1 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
  if (ws != nullptr && !ws_aligned(ws)) return SGEMM_ERR_WORKSPACE;
  if (M == 0 || N == 0 || batch == 0) return SGEMM_OK;
  const bool no_product = (alpha == 0.0f || K == 0);
  if (no_product && beta == 1.0f) return SGEMM_OK;
  Problem p{M,  N,  K,  alpha, beta, A, lda, B, ldb, C, ldc, opA == SGEMM_OP_T, opB == SGEMM_OP_T,
            sa, sb, sc, batch, ws, ws != nullptr ? ws_bytes : 0ULL};
  const int v = no_product ? -1
                           : ((variant >= 0) ? variant
                                             : choose_variant(p, g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED));
  // Every launch is checked before the first is enqueued (host only).
  if (!plan_fits(p, v, no_product)) return SGEMM_ERR_GRID;
  st = check_device();
  if (st != SGEMM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_all(p, v, no_product, s) != 0 || launch_plan().failed) {
    launch_plan().failed = false;
    return SGEMM_ERR_LAUNCH;  // not reached: the plan above fitted
  }
  return (hipGetLastError() == hipSuccess) ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int select(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
           long long sa, const float *B, int ldb, long long sb, float beta, const float *C, int ldc,
           long long sc, int batch, unsigned long long ws_bytes = 0) {
  const int st = check_args(opA, opB, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0 || batch == 0 || alpha == 0.0f || K == 0) return kNoKernel;
  // (a stand-in workspace address: only its presence and size matter here)
  const Problem p{M,   N,   K,   alpha, beta, A, lda, B, ldb, const_cast<float *>(C), ldc,
                  opA == SGEMM_OP_T, opB == SGEMM_OP_T, sa, sb, sc, batch,
                  ws_bytes ? reinterpret_cast<void *>(256) : nullptr, ws_bytes};
  const int v = choose_variant(p, g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED);
  return plan_fits(p, v, false) ? v : SGEMM_ERR_GRID;
}

// Workspace variant v uses on this problem (0: none); the edge split's two
// launches run one after the other and share it.
long long variant_ws_bytes(const Problem &p, int v) {
  if (v == kSkinnyFixed) return skinny_fixed_bytes(p);
  if (v == kSkinnyWs) return skinny_split_bytes(p);
  if (v == kFewRowsWs) return fewrows_split_bytes(p);
  if (v == kEdgeSplit) {
    const bool atomics = g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED;
    const EdgePlan ep = edge_plan(p);
    if (ep.side < 0) return variant_ws_bytes(p, choose_variant(p, atomics));
    const Problem bulk = edge_part(p, ep.side, ep.keep, false);
    long long need = variant_ws_bytes(bulk, choose_variant(bulk, atomics));
    Problem parts[2];
    const int np = thin_parts(p, ep.side, ep.keep, parts);
    for (int i = 0; i < np; ++i) {
      const long long b = variant_ws_bytes(parts[i], choose_variant(parts[i], atomics));
      if (b > need) need = b;
    }
    return need;
  }
  for (const TailFamily &tf : kTailFamilies)
    if (tf.variant == v) return family_tail_plan(tf, p).bytes;
  return 0;
}

// Workspace the automatic choice of the workspace entry points would use for
// this problem (0: none), or a negative status for invalid sizes.
long long workspace_size(int opA, int opB, int M, int N, int K, int batch) {
  if ((opA != SGEMM_OP_N && opA != SGEMM_OP_T) || (opB != SGEMM_OP_N && opB != SGEMM_OP_T))
    return SGEMM_ERR_OP;
  if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_ERR_DIM;
  if (M == 0 || N == 0 || K == 0 || batch != 1) return 0;
  const float *fake = reinterpret_cast<const float *>(256);
  const int lda = opA == SGEMM_OP_T ? M : K, ldb = opB == SGEMM_OP_T ? K : N;
  const Problem p{M,    N,   K,   1.0f, 0.0f, fake, lda, fake, ldb, const_cast<float *>(fake), N,
                  opA == SGEMM_OP_T, opB == SGEMM_OP_T, 0, 0, 0, 1,
                  reinterpret_cast<void *>(256), (unsigned long long)kTailWorkspaceBytes};
  return variant_ws_bytes(p, choose_variant(p, g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED));
}

// Scratch of the entry point that allocates nothing
// (sgemm_strided_batched_noalloc): the workspace of the split tail form as a
// file-scope device array, 4 KiB of counters plus 32 MiB of partial tiles --
// the most any problem's split can use.  Every GPU the library runs on holds
// its own copy from module load to process end.  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, once, with that device current.
constexpr unsigned long long kScratchBytes = (unsigned long long)kTailWorkspaceBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device; set once

// The device address of this device's scratch (set up on the first call on
// the device), or nullptr when the runtime cannot give it.  The counters
// must start at zero: the array is zero at load, every call that uses it
// leaves them zero, and the set-up clears them once more with a kernel on
// `s` (a kernel, not a memset, so a captured first call replays cleanly).
void *device_scratch(int dev, hipStream_t s) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    // zero the counters: kTailFlagBytes of zero floats (zero bits) through
    // the C-scaling kernel with beta = 0
    Problem z{};
    z.M = 1;
    z.N = (int)(kTailFlagBytes / 4);
    z.beta = 0.0f;
    z.C = reinterpret_cast<float *>(ptr);
    z.ldc = z.N;
    z.batch = 1;
    if (launch_scale(z, s) != 0 || hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int run_noalloc(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                long long sa, const float *B, int ldb, long long sb, float beta, float *C, int ldc,
                long long sc, int batch, void *stream) {
  int st = check_args(opA, opB, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch);
  if (st != SGEMM_OK) return st;
  if (M == 0 || N == 0 || batch == 0) return SGEMM_OK;
  // The scratch a call may use: the split plan of the variant the choice
  // takes with kScratchBytes available (never more, as plans are capped at
  // the workspace maximum); a call that would need more is refused.
  if (alpha != 0.0f && K > 0) {
    const Problem p{M,   N,   K,   alpha, beta, A, lda, B, ldb, C, ldc, opA == SGEMM_OP_T, opB == SGEMM_OP_T,
                    sa,  sb,  sc,  batch, reinterpret_cast<void *>(256), kScratchBytes};
    const int v = choose_variant(p, g_atomics_mode.load() == SGEMM_ATOMICS_ALLOWED);
    for (const TailFamily &tf : kTailFamilies)
      if (tf.variant == v && (unsigned long long)family_tail_plan(tf, p).bytes > kScratchBytes)
        return SGEMM_ERR_WORKSPACE;
  }
  st = check_device();
  if (st != SGEMM_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SGEMM_ERR_DEVICE;
  void *ws = device_scratch(dev, reinterpret_cast<hipStream_t>(stream));
  if (ws == nullptr) return SGEMM_ERR_LAUNCH;
  return run(opA, opB, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch, ws, kScratchBytes,
             stream, -1);
}

}  // namespace
}  // namespace sg950

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, void *stream) {
  return sg950::run(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1,
                    nullptr, 0, stream, -1);
}

int sgemm_ex(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream, int variant) {
  return sg950::run(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1,
                    nullptr, 0, stream, variant);
}

int sgemm_op(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, void *stream) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr, 0,
                    stream, -1);
}

int sgemm_op_ex(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, void *stream, int variant) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr, 0,
                    stream, variant);
}

int sgemm_strided_batched(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                          int lda, long long strideA, const float *B, int ldb, long long strideB,
                          float beta, float *C, int ldc, long long strideC, int batch,
                          void *stream) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                    strideC, batch, nullptr, 0, stream, -1);
}

int sgemm_strided_batched_ex(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                             int lda, long long strideA, const float *B, int ldb,
                             long long strideB, float beta, float *C, int ldc, long long strideC,
                             int batch, void *stream, int variant) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                    strideC, batch, nullptr, 0, stream, variant);
}

int sgemm_strided_batched_ws(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                             int lda, long long strideA, const float *B, int ldb, long long strideB,
                             float beta, float *C, int ldc, long long strideC, int batch,
                             void *workspace, unsigned long long workspace_bytes, void *stream) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                    strideC, batch, workspace, workspace_bytes, stream, -1);
}

int sgemm_strided_batched_ws_ex(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                                int lda, long long strideA, const float *B, int ldb,
                                long long strideB, float beta, float *C, int ldc, long long strideC,
                                int batch, void *workspace, unsigned long long workspace_bytes,
                                void *stream, int variant) {
  return sg950::run(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                    strideC, batch, workspace, workspace_bytes, stream, variant);
}

int sgemm_strided_batched_ws_select_variant(int opA, int opB, int M, int N, int K, float alpha,
                                            const float *A, int lda, long long strideA,
                                            const float *B, int ldb, long long strideB, float beta,
                                            const float *C, int ldc, long long strideC, int batch,
                                            unsigned long long workspace_bytes) {
  return sg950::select(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                       strideC, batch, workspace_bytes);
}

int sgemm_strided_batched_noalloc(int opA, int opB, int M, int N, int K, float alpha,
                                  const float *A, int lda, long long strideA, const float *B,
                                  int ldb, long long strideB, float beta, float *C, int ldc,
                                  long long strideC, int batch, void *stream) {
  return sg950::run_noalloc(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                            strideC, batch, stream);
}

long long sgemm_workspace_size(int opA, int opB, int M, int N, int K, int batch) {
  return sg950::workspace_size(opA, opB, M, N, K, batch);
}

int sgemm_num_variants(void) { return sg950::kNumVariants; }

const char *sgemm_variant_name(int variant) {
  if (variant < 0 || variant >= sg950::kNumVariants) return "";
  return sg950::kVariants[variant].name;
}

int sgemm_select_variant(int M, int N, int K, float alpha, const float *A, int lda,
                         const float *B, int ldb, float beta, const float *C, int ldc) {
  return sg950::select(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc,
                       0, 1);
}

int sgemm_op_select_variant(int opA, int opB, int M, int N, int K, float alpha, const float *A,
                            int lda, const float *B, int ldb, float beta, const float *C, int ldc) {
  return sg950::select(opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1);
}

int sgemm_strided_batched_select_variant(int opA, int opB, int M, int N, int K, float alpha,
                                         const float *A, int lda, long long strideA,
                                         const float *B, int ldb, long long strideB, float beta,
                                         const float *C, int ldc, long long strideC, int batch) {
  return sg950::select(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                       strideC, batch);
}

const char *sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "success";
    case SGEMM_ERR_DIM: return "invalid dimension (negative M, N, K or batch)";
    case SGEMM_ERR_LD: return "invalid leading dimension (shorter than the stored row it spans)";
    case SGEMM_ERR_PTR: return "NULL matrix pointer";
    case SGEMM_ERR_LAUNCH: return "kernel launch failed";
    case SGEMM_ERR_DEVICE: return "current device is not an MI355X (gfx950)";
    case SGEMM_ERR_VARIANT: return "variant index out of range";
    case SGEMM_ERR_OP: return "invalid operation (opA and opB must be SGEMM_OP_N or SGEMM_OP_T)";
    case SGEMM_ERR_STRIDE: return "invalid batch stride (negative, or slices of C overlap)";
    case SGEMM_ERR_GRID: return "problem too large for the launch grid of its kernel (nothing was enqueued)";
    case SGEMM_ERR_WORKSPACE:
      return "workspace not 16-byte aligned, or the call needs more scratch than the library's static buffer";
    default: return "unknown status";
  }
}

int sgemm_version(void) { return 5; }

int sgemm_set_atomics_mode(int mode) {
  if (mode != SGEMM_ATOMICS_ALLOWED && mode != SGEMM_ATOMICS_NOT_ALLOWED) return SGEMM_ERR_OP;
  sg950::g_atomics_mode.store(mode);
  return SGEMM_OK;
}

int sgemm_get_atomics_mode(void) { return sg950::g_atomics_mode.load(); }

}  // extern "C"
