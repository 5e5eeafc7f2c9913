// sgemm_mfma8.hip -- matrix-core variants with eight waves on a 128x128 or
// 64x64 tile (two waves per SIMD).  With up to a few hundred tiles -- one or
// two per CU, e.g. 1024^3 to 2048^3 -- a four-wave workgroup leaves a single
// wave per SIMD, which cannot cover the LDS and global-memory latencies by
// itself; a second wave on each SIMD does.  The kernel template is in
// sgemm_mfma.hpp.
#include "sgemm_mfma.hpp"

namespace sg950 {

//                  name                              MI   BM   BN  BK  WM WN MINW BPAD PIPE  SPLITK
SG950_MFMA_LAUNCHER(mfma32_128x128x32_4x2,            32, 128, 128, 32, 4, 2, 2, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_128x128x64_4x2,            32, 128, 128, 64, 4, 2, 2, 4, false, false)
SG950_MFMA_LAUNCHER(mfma16_64x64x64_4x2_pipe,         16,  64,  64, 64, 4, 2, 2, 4, true,  false)
SG950_MFMA_LAUNCHER(mfma32_128x128x32_4x2_splitk,     32, 128, 128, 32, 4, 2, 2, 4, false, true)
SG950_MFMA_LAUNCHER(mfma16_64x64x64_4x2_pipe_splitk,  16,  64,  64, 64, 4, 2, 2, 4, true,  true)

}  // namespace sg950
