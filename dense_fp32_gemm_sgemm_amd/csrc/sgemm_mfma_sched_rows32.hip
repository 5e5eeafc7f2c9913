// sgemm_mfma_sched_rows32.hip -- 32x64 tiles on the ordered slab loop
// (sgemm_sched.hpp), for row counts a 64-row tile would leave partly empty.
//
// A product with M just past a multiple of 64 (96, 160, 224, 352 ...) spends
// up to half of its last row of 64-row tiles on rows outside C.  With 32-row
// tiles every row computed is a row of C.  The tile is 32x64 with four waves
// (2 x 2, 16x32 wave tiles of 16x16 blocks), 64-deep slabs and 51 KiB of
// LDS, so three workgroups share a CU; its steady rate is below the 64x64
// tile's (127 against 131-135 TFLOP/s at 4096^3 on MI355X), so the automatic
// choice takes it only where the better row fill pays.  The split form runs
// K ranges on separate workgroups and adds them with atomics after a
// beta-scaling launch, for shapes with too few tiles to give every CU work.
// With A not transposed the tile also serves M below 32 (rows past M read
// row M - 1 of A and are not stored), so that 17 to 31 rows of a large B run
// on it as well.  When the ordered loop's preconditions fail (K shorter than
// one slab, N below 64, or M below 32 with A transposed) both fall back to
// the 64x64 variants, which accept every problem.
#include "sgemm_sched.hpp"

namespace sg950 {

int launch_mfma16_32x64x64_2x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<16, 32, 64, 64, 2, 2, 2, 4, false, true>(p, s, launch_mfma16_64x64x64_4x2_sched);
}

int launch_mfma16_32x64x64_2x2_sched_splitk(const Problem &p, hipStream_t s) {
  return launch_sched<16, 32, 64, 64, 2, 2, 2, 4, true, true>(p, s, launch_mfma16_64x64x64_4x2_pipe_splitk);
}

}  // namespace sg950
