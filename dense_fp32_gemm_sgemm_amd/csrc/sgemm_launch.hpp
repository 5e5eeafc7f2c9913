// sgemm_launch.hpp -- host-side launchers of the SGEMM kernel families.
//
// Each launcher enqueues one GEMM on `stream` and returns 0, or -1 when the
// problem's grid would exceed the launch limits.  Arguments are already
// validated by the C entry points (sizes >= 1, leading dimensions in range,
// pointers non-NULL, alpha != 0, K >= 1).
#pragma once

#include <hip/hip_runtime.h>

#include "sgemm_common.hpp"

namespace sg950 {

// Every launcher covers all p.batch slices of the problem (grid z = batch,
// at most 65535; the entry points split larger batches).
int launch_simple(const Problem &p, hipStream_t stream);
// C = beta*C over every batch slice (zeros without reading C when beta == 0).
int launch_scale(const Problem &p, hipStream_t stream);

// Register-tiled VALU kernel: 128x256 tile, 8x16 outputs per thread.
int launch_valu_128x256(const Problem &p, hipStream_t stream);

// Matrix-core kernels, named <instruction>_<BM>x<BN>x<BK>_<waves M>x<waves N>;
// _pipe: software-pipelined slab order; _w4: registers capped for four waves
// per SIMD.
int launch_mfma32_256x256x32_4x2(const Problem &p, hipStream_t stream);
int launch_mfma32_256x256x16_4x2(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x32_2x2(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x32_2x2_pipe(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x16_2x2_w4(const Problem &p, hipStream_t stream);
int launch_mfma32_64x64x16_1x1(const Problem &p, hipStream_t stream);
int launch_mfma16_128x128x16_2x2(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x16_2x2(const Problem &p, hipStream_t stream);
// _splitk: K split over blockIdx.y when the tiles alone cannot fill the GPU;
// C is scaled by beta first and the partial products are added with float
// atomics (summation order of the splits unspecified).
int launch_mfma32_128x128x32_2x2_splitk(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x16_2x2_splitk(const Problem &p, hipStream_t stream);
int launch_mfma32_64x64x16_1x1_splitk(const Problem &p, hipStream_t stream);
// Eight waves (4x2) on 128x128 and 64x64 tiles, two waves per SIMD
// (sgemm_mfma8.hip).
int launch_mfma32_128x128x32_4x2(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x64_4x2(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x64_4x2_pipe(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x32_4x2_splitk(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x64_4x2_pipe_splitk(const Problem &p, hipStream_t stream);
// _sched: the explicitly ordered slab loop (sgemm_mfma_sched.hip) when K is a
// multiple of the slab depth, the tile fits in C and both operands allow
// 16-byte loads; otherwise the same tile family on the plain loop.
int launch_mfma32_256x256x32_2x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma32_256x256x32_4x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma32_128x128x32_4x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x64_4x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma16_128x128x64_4x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x64_4x2_sched_splitk(const Problem &p, hipStream_t stream);
int launch_mfma16_128x128x32_2x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma16_128x64x64_4x2_sched(const Problem &p, hipStream_t stream);
// 32x64 tiles (four waves, three workgroups per CU) for row counts just past
// a multiple of 64, unsplit and with K split over workgroups.
int launch_mfma16_32x64x64_2x2_sched(const Problem &p, hipStream_t stream);
int launch_mfma16_32x64x64_2x2_sched_splitk(const Problem &p, hipStream_t stream);

// The same families with the fixed-order split of their last, partial round
// of tiles (needs a workspace in the Problem; otherwise the plain loop).
int launch_mfma16_128x128x32_2x2_sched_tail(const Problem &p, hipStream_t stream);
int launch_mfma16_128x128x64_4x2_sched_tail(const Problem &p, hipStream_t stream);
int launch_mfma16_128x64x64_4x2_sched_tail(const Problem &p, hipStream_t stream);
int launch_mfma16_64x64x64_4x2_sched_tail(const Problem &p, hipStream_t stream);

// Few rows of C (M <= 8): streams B across every CU, K split over
// workgroups, float atomics into C (scaled by beta first).  Returns -1 for
// M > 8.
int launch_skinny(const Problem &p, hipStream_t stream);

// Few rows of C (M <= 8), one batch slice, B untransposed, with a workspace:
// B streamed in 1 KiB row segments by (column strip, K chunk) workgroups, the
// chunks' partial strips added in a fixed order by the strip's last chunk
// (one launch, no atomics on C).  Without a workspace that holds
// skinny_fixed_bytes(p), or where the form does not apply, launch_skinny.
// Returns -1 for M > 8.
int launch_skinny_fixed(const Problem &p, hipStream_t stream);
// Workspace bytes that form needs for p (0: the form does not apply).
long long skinny_fixed_bytes(const Problem &p);

// Few rows of C (M <= 8), one batch slice, B untransposed, with a workspace:
// the full-K strip kernel with K split over up to four ranges when its strips
// alone give fewer workgroups than CUs (partial strips added in range order
// by the last range); otherwise launch_skinny.  Returns -1 for M > 8.
int launch_skinny_ws(const Problem &p, hipStream_t stream);
// Workspace bytes of that split (0: it does not apply).
long long skinny_split_bytes(const Problem &p);

// Few columns of C (N <= 16): streams A, the matrix cores accumulate 16 x 16
// blocks, K split over the waves of a workgroup, one launch.  Returns -1 for
// N > 16.
int launch_narrow(const Problem &p, hipStream_t stream);

// Few rows of C (M <= 32): streams B, the matrix cores accumulate 16 x 16
// blocks, K split over the waves of a workgroup, one launch.  Returns -1 for
// M outside 1..32.
int launch_fewrows(const Problem &p, hipStream_t stream);

// The same kernel, one batch slice, with a workspace: at most 128 column
// strips (16, 32 or 64 columns; up to 8192 columns in all), each split into
// two to four K chunks so that strips x chunks fill at most one workgroup
// per CU, the chunks' partial blocks added in chunk order by the strip's
// last chunk; otherwise launch_fewrows.  Returns -1 for M outside 1..32.
int launch_fewrows_ws(const Problem &p, hipStream_t stream);
// Workspace bytes of that split (0: it does not apply).
long long fewrows_split_bytes(const Problem &p);
// How full (percent) the last round of 256 workgroups is on the unsplit
// kernel's grid, and the columns of its strips (16, 32 or 64).
int fewrows_round_fill_pct(const Problem &p);
int fewrows_strip_cols(const Problem &p);

// Operand alignment classes of the plain-loop and VALU kernels, which read
// vectors through 16-byte typed pointers: an operand may be read with
// 16-byte vector loads when its base is 16-byte aligned and its leading
// dimension is a multiple of four; when its rows run along M or N (A
// transposed, B not) the row length must be one too, so a vector never
// crosses the end of a row.  (The ordered-loop and streaming kernels copy
// their vectors instead, which needs only 4-byte alignment: the global loads
// and stores themselves need no more.)
inline bool a_vec_ok(const Problem &p) {
  return ((reinterpret_cast<uintptr_t>(p.A) & 15) == 0) && (p.lda % 4 == 0) &&
         (!p.ta || p.M % 4 == 0) && (p.batch <= 1 || p.sa % 4 == 0);
}
inline bool b_vec_ok(const Problem &p) {
  return ((reinterpret_cast<uintptr_t>(p.B) & 15) == 0) && (p.ldb % 4 == 0) &&
         (p.tb || p.N % 4 == 0) && (p.batch <= 1 || p.sb % 4 == 0);
}
inline bool c_vec_ok(const Problem &p) {
  return ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 4 == 0) && (p.N % 4 == 0) &&
         (p.batch <= 1 || p.sc % 4 == 0);
}

}  // namespace sg950
