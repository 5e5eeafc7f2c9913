// sgemm_mfma_sched.hip -- the variants on sched_kernel (sgemm_sched.hpp).
// Each launches the scheduled kernel when the problem meets its
// preconditions and otherwise the variant of the same tile family built on
// mfma_kernel, so that every variant accepts every problem.
#include "sgemm_sched.hpp"

namespace sg950 {

// 256x256 tile, four waves (one per SIMD) with 128x128 wave tiles.
int launch_mfma32_256x256x32_2x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<32, 256, 256, 32, 2, 2, 1, 4>(p, s, launch_mfma32_256x256x32_4x2);
}
// 256x256 tile, eight waves (two per SIMD) with 64x128 wave tiles.
int launch_mfma32_256x256x32_4x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<32, 256, 256, 32, 4, 2, 2, 4>(p, s, launch_mfma32_256x256x32_4x2);
}
// 128x128 tile, eight waves with 32x64 wave tiles.
int launch_mfma32_128x128x32_4x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<32, 128, 128, 32, 4, 2, 2, 4>(p, s, launch_mfma32_128x128x32_4x2);
}
// 128x128 tile, eight waves with 32x64 wave tiles of 16x16 blocks, 64-deep
// slabs (half the barriers of the 32-deep form; one workgroup per CU).
int launch_mfma16_128x128x64_4x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 128, 64, 4, 2, 2, 4>(p, s, launch_mfma32_128x128x32_4x2_sched);
}
// 128x128 tile, four waves with 64x64 wave tiles of 16x16 blocks, 32-deep
// slabs: 69 KiB of LDS, so two workgroups share a CU when there are at least
// two tiles per CU.
int launch_mfma16_128x128x32_2x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 128, 32, 2, 2, 1, 4>(p, s, launch_mfma32_128x128x32_4x2);
}
// 128x64 tile, eight waves with 32x32 wave tiles of 16x16 blocks, 64-deep
// slabs: one tile per CU for problems with half as many 128x128 tiles.
int launch_mfma16_128x64x64_4x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<16, 128, 64, 64, 4, 2, 2, 4>(p, s, launch_mfma16_64x64x64_4x2_sched);
}
// The same tile with K split over workgroups when the tiles cannot give the
// CUs two workgroups each.
int launch_mfma16_64x64x64_4x2_sched_splitk(const Problem &p, hipStream_t s) {
  return launch_sched<16, 64, 64, 64, 4, 2, 2, 4, true>(p, s, launch_mfma16_64x64x64_4x2_pipe_splitk);
}
// 64x64 tile, eight waves with 16x32 wave tiles, 64-deep slabs.
int launch_mfma16_64x64x64_4x2_sched(const Problem &p, hipStream_t s) {
  return launch_sched<16, 64, 64, 64, 4, 2, 2, 4>(p, s, launch_mfma16_64x64x64_4x2_pipe);
}

}  // namespace sg950
