// sgemm_mfma.hip -- the matrix-core variants with one wave per SIMD per
// workgroup slot (four-wave 128x128 and 64x64 tiles) and the eight-wave
// 256x256 tiles of the large-problem path.  The kernel template is in
// sgemm_mfma.hpp; each line below instantiates one variant (every operand
// orientation and alignment class) behind the launcher the variant table
// calls.
#include "sgemm_mfma.hpp"

namespace sg950 {

//                  name                          MI   BM   BN  BK  WM WN MINW BPAD PIPE  SPLITK
SG950_MFMA_LAUNCHER(mfma32_256x256x32_4x2,        32, 256, 256, 32, 4, 2, 2, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_256x256x16_4x2,        32, 256, 256, 16, 4, 2, 2, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_128x128x32_2x2,        32, 128, 128, 32, 2, 2, 1, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_128x128x32_2x2_pipe,   32, 128, 128, 32, 2, 2, 1, 4, true,  false)
SG950_MFMA_LAUNCHER(mfma32_128x128x16_2x2_w4,     32, 128, 128, 16, 2, 2, 4, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_64x64x16_1x1,          32,  64,  64, 16, 1, 1, 1, 4, false, false)
SG950_MFMA_LAUNCHER(mfma16_128x128x16_2x2,        16, 128, 128, 16, 2, 2, 1, 4, false, false)
SG950_MFMA_LAUNCHER(mfma16_64x64x16_2x2,          16,  64,  64, 16, 2, 2, 1, 4, false, false)
SG950_MFMA_LAUNCHER(mfma32_128x128x32_2x2_splitk, 32, 128, 128, 32, 2, 2, 1, 4, false, true)
SG950_MFMA_LAUNCHER(mfma16_64x64x16_2x2_splitk,   16,  64,  64, 16, 2, 2, 1, 4, false, true)
SG950_MFMA_LAUNCHER(mfma32_64x64x16_1x1_splitk,   32,  64,  64, 16, 1, 1, 1, 4, false, true)

}  // namespace sg950
