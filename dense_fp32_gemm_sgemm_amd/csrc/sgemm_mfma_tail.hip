// sgemm_mfma_tail.hip -- ordered-loop tile families with the fixed-order
// split of the last round of tiles (sched_kernel's TAIL form,
// sgemm_sched.hpp).
//
// A grid whose tiles do not fill the CUs' workgroup slots a whole number of
// times leaves most CUs idle in its last round: (4095, 4097, 1023) on 128x128
// tiles is 1056 tiles for 512 slots, two full rounds and 32 tiles.  Here the
// whole rounds run as usual and each tile of the last round is split into K
// ranges, one workgroup each, so that the last round fills the slots too;
// the partial tiles go to a caller-provided workspace and the workgroup that
// finishes a tile's ranges last adds them in range order and stores the
// tile.  Every output is still one fixed sum, so repeated calls give bitwise
// the same C (no atomics on C).  The pages point at splitting K when the
// output tiles cannot fill the GPU ("The road to a fast GEMM", "Where to go
// next").  Without a workspace (or with a batch), and when the rounds are
// whole, each variant runs its family's ordinary loop.  (The 256x256 family
// has no tail form: with 256 accumulators per lane its loop has no registers
// to spare for the partial-tile epilogue, which then spilled and slowed the
// whole kernel on MI355X.)
#include "sgemm_sched.hpp"

namespace sg950 {

// 128x128 tile, four waves (64x64 wave tiles of 16x16 blocks), 32-deep
// slabs, two workgroups per CU.
int launch_mfma16_128x128x32_2x2_sched_tail(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 128, 32, 2, 2, 1, 4, false, false, true, 2>(p, s, launch_mfma32_128x128x32_4x2);
}
// 128x128 tile, eight waves, 64-deep slabs, one workgroup per CU.
int launch_mfma16_128x128x64_4x2_sched_tail(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 128, 64, 4, 2, 2, 4, false, false, true, 1>(p, s,
                                                                            launch_mfma32_128x128x32_4x2_sched);
}
// 128x64 tile, eight waves, 64-deep slabs, one workgroup per CU.
int launch_mfma16_128x64x64_4x2_sched_tail(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 64, 64, 4, 2, 2, 4, false, false, true, 1>(p, s, launch_mfma16_64x64x64_4x2_sched);
}
// 64x64 tile, eight waves, 64-deep slabs, two workgroups per CU.
int launch_mfma16_64x64x64_4x2_sched_tail(const Problem &p, hipStream_t s) {
  return launch_sched<16, 64, 64, 64, 4, 2, 2, 4, false, false, true, 2>(p, s, launch_mfma16_64x64x64_4x2_pipe);
}

}  // namespace sg950
