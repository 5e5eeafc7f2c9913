"""CPU tests of the C boundary: the library loads, exports what the headers
declare, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_fp32_gemm_sgemm_amd as sg
from dense_fp32_gemm_sgemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("sgemm.h", "sgemm_ceiling.h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY):
        from dense_fp32_gemm_sgemm_amd import _build
        _build.build()
    return _lib.load()


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(sgemm\w*)\s*\(", text, flags=re.M)
    return names


def test_headers_declare_the_entry_points():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(lib, name):
    assert hasattr(lib, name), name


def test_exported_symbols_are_c_linkage(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (sgemm\w*)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_variant_registry(lib):
    n = sg.sgemm_num_variants()
    names = sg.variant_names()
    assert n == len(names) >= 3 and len(set(names)) == n
    assert names[0] == "simple"
    assert any(x.startswith("mfma32") for x in names) and any(x.startswith("valu") for x in names)
    assert sg.sgemm_variant_name(n) == "" and sg.sgemm_variant_name(-1) == ""
    assert sg.sgemm_version() == 5


FAKE = 0x1000  # never dereferenced: every call below fails or returns before any HIP call


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_DIM),
    ((4, -1, 4, 1.0, FAKE, 4, FAKE, 1, 0.0, FAKE, 1), sg.SGEMM_ERR_DIM),
    ((4, 4, -2, 1.0, FAKE, 1, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_DIM),
    ((4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_LD),
    ((4, 4, 8, 1.0, FAKE, 8, FAKE, 3, 0.0, FAKE, 4), sg.SGEMM_ERR_LD),
    ((4, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 3), sg.SGEMM_ERR_LD),
    ((4, 4, 0, 1.0, None, 0, None, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_LD),   # lda >= 1
    ((4, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, None, 4), sg.SGEMM_ERR_PTR),
    ((4, 4, 8, 1.0, None, 8, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_PTR),
    ((4, 4, 8, 1.0, FAKE, 8, None, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_PTR),
    ((0, 4, 8, 1.0, None, 8, None, 4, 0.0, None, 4), sg.SGEMM_OK),      # M == 0: no-op
    ((4, 0, 8, 1.0, None, 8, None, 1, 0.0, None, 1), sg.SGEMM_OK),      # N == 0: no-op
    ((4, 4, 8, 0.0, None, 8, None, 4, 1.0, FAKE, 4), sg.SGEMM_OK),      # alpha 0, beta 1
    ((4, 4, 0, 2.0, None, 1, None, 4, 1.0, FAKE, 4), sg.SGEMM_OK),      # K 0, beta 1
])
def test_argument_checks_before_any_hip_call(lib, args, status):
    assert sg.sgemm(*args, 0) == status
    assert sg.sgemm_ex(*args, 0, -1) == status


def test_variant_index_checked(lib):
    args = (4, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 4)
    n = sg.sgemm_num_variants()
    assert sg.sgemm_ex(*args, 0, n) == sg.SGEMM_ERR_VARIANT
    assert sg.sgemm_ex(*args, 0, -2) == sg.SGEMM_ERR_VARIANT


@pytest.mark.parametrize("ops,args,status", [
    ((2, 0), (4, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_OP),
    ((0, -1), (4, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 4), sg.SGEMM_ERR_OP),
    ((1, 0), (4, 6, 8, 1.0, FAKE, 3, FAKE, 6, 0.0, FAKE, 6), sg.SGEMM_ERR_LD),  # A^T: lda >= M
    ((1, 0), (4, 6, 8, 1.0, FAKE, 4, FAKE, 6, 0.0, FAKE, 6), "valid"),
    ((0, 1), (4, 6, 8, 1.0, FAKE, 8, FAKE, 7, 0.0, FAKE, 6), sg.SGEMM_ERR_LD),  # B^T: ldb >= K
    ((1, 1), (0, 6, 8, 1.0, None, 1, None, 8, 0.0, None, 6), sg.SGEMM_OK),
    ((1, 1), (4, 6, 8, 1.0, FAKE, 4, None, 8, 0.0, FAKE, 6), sg.SGEMM_ERR_PTR),
])
def test_op_argument_checks(lib, ops, args, status):
    if status == "valid":   # a valid problem: the choice is a variant index
        st = sg.sgemm_op_select_variant(*ops, *args)
        assert 0 <= st < sg.sgemm_num_variants()
        return
    assert sg.sgemm_op(*ops, *args, 0) == status
    assert sg.sgemm_op_ex(*ops, *args, 0, -1) == status


def test_op_select_avoids_few_rows_kernel_for_transposed_b(lib):
    n = sg.sgemm_variant_name
    assert n(sg.sgemm_op_select_variant(0, 0, 1, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE,
                                        4096)) == "skinny_m8"
    assert n(sg.sgemm_op_select_variant(0, 1, 1, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE,
                                        4096)) != "skinny_m8"
    assert n(sg.sgemm_op_select_variant(1, 1, 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0,
                                        FAKE, 4096)).startswith("mfma32_256x256")
    assert n(sg.sgemm_op_select_variant(0, 1, 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0,
                                        FAKE, 4096)) == "mfma32_256x256x32_2x2_sched"


@pytest.mark.parametrize("args,status", [
    # opA opB M N K alpha A lda sA B ldb sB beta C ldc sC batch
    ((0, 0, 4, 4, 8, 1.0, FAKE, 8, 32, FAKE, 4, 32, 0.0, FAKE, 4, 16, -1), sg.SGEMM_ERR_DIM),
    ((0, 0, 4, 4, 8, 1.0, FAKE, 8, -1, FAKE, 4, 32, 0.0, FAKE, 4, 16, 2), sg.SGEMM_ERR_STRIDE),
    ((0, 0, 4, 4, 8, 1.0, FAKE, 8, 32, FAKE, 4, 32, 0.0, FAKE, 4, 15, 2), sg.SGEMM_ERR_STRIDE),
    ((0, 0, 4, 4, 8, 1.0, FAKE, 8, 32, FAKE, 4, 32, 0.0, FAKE, 4, 0, 1), "valid"),   # one slice
    ((0, 0, 4, 4, 8, 1.0, FAKE, 8, 0, FAKE, 4, 0, 0.0, FAKE, 4, 16, 9), "valid"),    # shared A, B
    ((0, 0, 4, 4, 8, 1.0, None, 8, 0, None, 4, 0, 0.0, None, 4, 16, 0), sg.SGEMM_OK),  # empty batch
    ((1, 0, 4, 4, 8, 1.0, FAKE, 3, 32, FAKE, 4, 32, 0.0, FAKE, 4, 16, 2), sg.SGEMM_ERR_LD),
    ((3, 0, 4, 4, 8, 1.0, FAKE, 8, 32, FAKE, 4, 32, 0.0, FAKE, 4, 16, 2), sg.SGEMM_ERR_OP),
])
def test_batched_argument_checks(lib, args, status):
    if status == "valid":
        st = sg.sgemm_strided_batched_select_variant(*args)
        assert 0 <= st < sg.sgemm_num_variants()
        return
    assert sg.sgemm_strided_batched(*args, 0) == status
    assert sg.sgemm_strided_batched_ex(*args, 0, -1) == status


def test_batched_select_counts_every_slice(lib):
    n = sg.sgemm_variant_name
    one = sg.sgemm_strided_batched_select_variant(0, 0, 512, 512, 512, 1.0, FAKE, 512, 512 * 512, FAKE,
                                                  512, 512 * 512, 0.0, FAKE, 512, 512 * 512, 1)
    many = sg.sgemm_strided_batched_select_variant(0, 0, 512, 512, 512, 1.0, FAKE, 512, 512 * 512,
                                                   FAKE, 512, 512 * 512, 0.0, FAKE, 512, 512 * 512, 64)
    assert n(one) == "mfma16_32x64x64_2x2_sched" and n(many).startswith("mfma32_256x256")


def _batched_choice(batch, M, N, K):
    return sg.sgemm_variant_name(sg.sgemm_strided_batched_select_variant(
        0, 0, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N, batch))


def test_batched_select_small_slices(lib):
    """Many small slices leave the one-lane kernel for tiled ones; tiles that
    would mostly lie outside a slice are not chosen."""
    assert _batched_choice(1, 127, 129, 17) == "simple"
    # few 64x64 tiles with a short K: 32x64 tiles (3.5 against 4.5 us, device time)
    assert _batched_choice(1, 128, 128, 128) == "mfma16_32x64x64_2x2_sched"
    assert _batched_choice(1, 256, 256, 65536) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _batched_choice(1024, 128, 128, 128) == "mfma32_128x128x16_2x2_w4"
    assert _batched_choice(256, 256, 256, 256) == "mfma32_256x256x32_2x2_sched"
    assert _batched_choice(4096, 32, 32, 32) == "mfma16_64x64x16_2x2_splitk"
    assert _batched_choice(128, 200, 300, 100) == "mfma16_64x64x16_2x2_splitk"
    assert _batched_choice(8, 1, 4096, 4096) == "skinny_m8"


def test_select_128_tiles(lib):
    """128x128 tiles: four waves (two workgroups per CU) once there are two
    tiles per CU, eight waves with 64-deep slabs when one round leaves each CU
    one tile; 128x128 over 256x256 tiles when the 256x256 tiles leave their
    last round mostly empty ((10000, 10000, 1000): 134 vs 120 TFLOP/s)."""
    assert _batched_choice(1, 8192, 1024, 8192) == "mfma16_128x128x32_2x2_sched"
    assert _batched_choice(1, 1024, 8192, 256) == "mfma16_128x128x32_2x2_sched"
    assert _batched_choice(1, 2048, 2048, 2048) == "mfma16_128x128x64_4x2_sched"
    assert _batched_choice(2, 2048, 2048, 2048) == "mfma16_128x128x32_2x2_sched"
    assert _batched_choice(1, 256, 16384, 4096) == "mfma16_128x128x64_4x2_sched"
    assert _batched_choice(1, 10000, 10000, 1000) == "edge_split"   # 16-row and -column edges: 136.9 vs 134.6


def test_select_last_round_tail(lib):
    """A tile count just past whole rounds of the 256 CUs leaves the last
    round nearly empty.  Where a thin edge of 1 to 16 rows or columns adds
    that row or column of tiles (1 to 32 rows or columns), the edge is split
    off to the few-columns or
    few-rows kernel and the bulk keeps the large tiles (measured, TFLOP/s:
    (4095, 4097, 1023) 129.9 against 118.9 on 64x64 tiles, (4095, 4097, 4095)
    143.8 vs 125.9, (2047, 2049, 2047) 121.7 vs 108.5 on 32x64, (8191, 1025,
    8191) 134.4 vs 118.8), in every orientation; otherwise smaller tiles win
    (3000^3 126 vs 104 on 128x128, (6144, 1024, 4096) 135 vs 108)."""
    for shape in ((4095, 4097, 4095), (8191, 1025, 8191), (2047, 4097, 4095), (4096, 4097, 1024),
                  (2047, 2049, 2047), (4097, 4095, 1023), (4097, 4097, 4097)):
        assert _batched_choice(1, *shape) == "edge_split", shape
    # row edges up to 32 go to the few-rows kernels ((4120, 4096, 2048) 143.3
    # against 122.9 TFLOP/s on 64x64 tiles, (2080, 2048, 2048) 128.1 vs 110.3)
    for shape in ((4120, 4096, 2048), (4128, 4096, 1024), (2080, 2048, 2048), (1056, 1024, 2048)):
        assert _batched_choice(1, *shape) == "edge_split", shape
    # column edges of 17 to 32 go as two few-columns strips ((4096, 4120,
    # 2048) 141.9 against 127.2 on 64x64 tiles, (4128, 4128, 2048) 137.3 vs
    # 128.4, (2048, 2080, 2048) 123.3 vs 114.7 on 32x64); (1024, 1056, 2048)
    # keeps 32x64 tiles (83.4 against 81.7 split)
    for shape in ((4128, 4128, 2048), (4096, 4120, 2048), (2048, 2080, 2048), (4095, 4127, 1023)):
        assert _batched_choice(1, *shape) == "edge_split", shape
    assert _batched_choice(1, 1024, 1056, 2048) != "edge_split"
    for ta in (0, 1):
        for tb in (0, 1):
            assert _op_choice(ta, tb, 4095, 4097, 1023) == "edge_split"
    # no thin edge (3000 = 11 x 256 + 184), or K below the fitted depths
    for shape in ((3000, 3000, 3000), (3072, 3072, 3072)):
        assert _batched_choice(1, *shape) == "mfma16_64x64x64_4x2_sched", shape
    assert _batched_choice(1, 1023, 8193, 257) == "mfma16_64x64x64_4x2_sched"
    assert _batched_choice(1, 6144, 1024, 4096) == "mfma16_128x64x64_4x2_sched"
    # whole rounds keep the large tiles
    assert _batched_choice(1, 4096, 4096, 1023) == "mfma32_256x256x32_2x2_sched"
    assert _batched_choice(1, 8192, 8192, 8192) == "mfma32_256x256x32_2x2_sched"


def test_select_rows_just_past_64(lib):
    """M just past a multiple of 64 leaves up to half of the last row of
    64-row tiles empty: 32x64 tiles, with K split over workgroups when the
    tiles cannot fill the CUs (measured, TFLOP/s: (96, 8192, 8192) 112.5
    against 92 on split 64x64 tiles, (96, 4096, 4096) 73.9 vs 68.4,
    (160, 4096, 4096) 88.8 vs 74.4, (320, 8192, 8192) 118.4 vs 111.3); at 32
    rows or fewer the few-rows kernels, and where 32-row tiles fill no better
    the 64x64 split."""
    r32 = "mfma16_32x64x64_2x2_sched"
    assert _op_choice(0, 0, 96, 8192, 8192) == r32 + "_splitk"
    assert _op_choice(0, 0, 96, 4096, 4096) == r32 + "_splitk"
    assert _op_choice(0, 0, 160, 4096, 4096) == r32 + "_splitk"
    assert _op_choice(0, 0, 320, 8192, 8192) == r32
    assert _op_choice(0, 0, 320, 4096, 4096) == r32
    assert _op_choice(0, 0, 48, 16384, 4096) == r32
    assert _op_choice(0, 0, 24, 1024, 4096) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 0, 352, 8192, 8192) == "mfma16_64x64x64_4x2_sched"


def test_select_narrow_problems(lib):
    """Few columns of C go to the few-columns kernel, few rows to the
    few-rows kernel or split-K tiles, never to the one-lane kernel (which
    leaves most of a wave idle when N is small)."""
    assert _batched_choice(1, 4096, 1, 4096) == "narrow_n16"
    assert _batched_choice(1, 65536, 8, 1024) == "narrow_n16"
    assert _batched_choice(1, 3000, 16, 100) == "narrow_n16"
    assert _batched_choice(1, 12, 15, 100000) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _batched_choice(1, 3, 4096, 4096) == "skinny_m8"
    assert _batched_choice(1, 8, 4096, 4096) == "fewrows_m32"
    assert _batched_choice(1, 9, 4096, 4096) == "fewrows_m32"
    assert _batched_choice(1, 5, 7, 9) == "simple"


def _op_choice(ta, tb, M, N, K, batch=1):
    lda = M if ta else K
    ldb = K if tb else N
    return sg.sgemm_variant_name(sg.sgemm_strided_batched_select_variant(
        ta, tb, M, N, K, 1.0, FAKE, lda, M * K, FAKE, ldb, K * N, 0.0, FAKE, N, M * N, batch))


def test_select_few_rows(lib):
    """Up to four rows of a moderate untransposed B on the vector-unit kernel,
    up to 32 rows on the matrix-core kernel when its column strips fill the
    CUs (with B transposed, above 16 rows only for wide strips or K <= 4096),
    split-K tiles otherwise; 17 to 32 rows with N*K >= 2^25 on 32-row tiles
    (below 32 rows only with A untransposed), and with B transposed from
    N*K >= 2^22 when K >= N (17 to 32 rows) or K >= 2N (9 to 16 rows)."""
    assert _op_choice(0, 0, 1, 4096, 4096) == "skinny_m8"
    assert _op_choice(0, 0, 4, 8192, 8192) == "skinny_m8"
    assert _op_choice(0, 0, 4, 16384, 16384) == "fewrows_m32"       # B too large for full-K strips
    assert _op_choice(0, 0, 4, 2048, 2048) == "fewrows_m32"
    assert _op_choice(0, 0, 1, 1024, 4096) == "fewrows_m32"
    assert _op_choice(0, 0, 12, 4096, 4096) == "fewrows_m32"
    assert _op_choice(1, 0, 32, 4096, 4096) == "fewrows_m32"
    # exactly 32 rows of a large B: 32-row tiles, split over K when few
    # ((32, 8192, 8192): 48.6 against 60.7 us on the few-rows kernel)
    assert _op_choice(0, 0, 32, 8192, 8192) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 1, 32, 4096, 16384) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 0, 32, 65536, 1024) == "mfma16_32x64x64_2x2_sched"
    try:
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_NOT_ALLOWED) == sg.SGEMM_OK
        assert _op_choice(0, 0, 32, 8192, 8192) == "fewrows_m32"
    finally:
        sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED)
    assert _op_choice(0, 0, 24, 1024, 4096) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 1, 16, 4096, 4096) == "fewrows_m32"
    assert _op_choice(0, 1, 16, 1024, 4096) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 1, 24, 4096, 4096) == "mfma16_32x64x64_2x2_sched_splitk"  # 20.9 vs 23.5 us
    assert _op_choice(0, 1, 32, 4096, 2048) == "fewrows_m32"  # N above K: 15.4 vs 16.4 us
    assert _op_choice(0, 0, 24, 4096, 4096) == "fewrows_m32"  # B untransposed below 2^25
    # fewer than 64 columns never go to the 32x64 tiles (they would not fit)
    assert _op_choice(0, 1, 24, 48, 100000) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 1, 12, 60, 200000) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 1, 24, 4096, 1024) == "fewrows_m32"
    assert _op_choice(1, 1, 24, 8192, 8192) == "fewrows_m32"  # A transposed: no short 32-row tile
    assert _op_choice(0, 1, 24, 8192, 8192) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 0, 20, 8192, 8192) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 1, 24, 4096, 16384) == "mfma16_32x64x64_2x2_sched_splitk"  # 49 vs 80 us
    assert _op_choice(1, 1, 24, 4096, 16384) == "mfma16_64x64x64_4x2_pipe_splitk"
    # 9 to 16 rows of a transposed B with K >= 2N: 32-row split tiles
    # ((16, 4096, 16384): 48.4 against 63.9 us); N above K/2 stays
    assert _op_choice(0, 1, 16, 4096, 16384) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 1, 12, 4096, 16384) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 1, 16, 16384, 16384) == "fewrows_m32"
    assert _op_choice(0, 1, 8, 4096, 16384) == "fewrows_m32"
    assert _op_choice(0, 0, 8, 512, 4096) == "skinny_m8"                # too few strips
    assert _op_choice(0, 0, 12, 1024, 256, batch=8) == "fewrows_m32"   # strips over the batch


def _ws_choice(ta, tb, M, N, K, ws_bytes=4096 + (32 << 20), batch=1):
    return sg.sgemm_variant_name(sg.sgemm_strided_batched_ws_select_variant(
        ta, tb, M, N, K, 1.0, FAKE, M if ta else K, M * K, FAKE, K if tb else N, K * N, 0.0, FAKE, N, M * N,
        batch, ws_bytes))


def test_select_few_rows_split_through_workspace(lib):
    """With a workspace, the matrix-core few-rows kernel split over K: up to
    16 rows from 1009 columns (64 strips of 16) at a K up to 32768, from fewer
    columns at a K up to 4096; above 16 rows where the unsplit kernel would be
    chosen.  Never beyond 2048 columns, never in a batch, never where the
    vector-unit strips split over K or 32-row tiles are chosen."""
    assert _ws_choice(0, 0, 8, 1024, 8192) == "fewrows_m32_ws"      # was the fixed-order VALU form
    assert _ws_choice(0, 0, 16, 1024, 8192) == "fewrows_m32_ws"     # was unsplit
    assert _ws_choice(0, 1, 4, 1024, 4096) == "fewrows_m32_ws"      # was split 64x64 tiles
    assert _ws_choice(0, 0, 1, 1500, 16384) == "fewrows_m32_ws"
    assert _ws_choice(1, 0, 12, 2048, 2048) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 8, 512, 4096) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 32, 2048, 4096) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 1, 2048, 4096) == "skinny_m8_ws"        # vector-unit strips split first
    assert _ws_choice(0, 0, 8, 8192, 4096) == "fewrows_m32"         # 256 strips of 32: a whole round
    assert _ws_choice(0, 0, 8, 4096, 4096) == "fewrows_m32_ws"      # unsplit strips of 16 columns
    assert _ws_choice(0, 0, 4, 4096, 4096) == "skinny_m8_ws"        # up to 4 rows: the VALU split
    assert _ws_choice(0, 1, 8, 3072, 4096) == "fewrows_m32"         # B transposed: unsplit past 2048
    # past 2048 columns, B untransposed, K >= 4096, the unsplit grid's last
    # round under 80% full (or, above four rows, its strips 16 columns wide):
    # the split on wider strips, ahead of the vector-unit strips split over
    # K; up to eight rows only while N*K <= 2^26
    assert _ws_choice(0, 0, 16, 6144, 4096) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 1, 3072, 8192) == "fewrows_m32_ws"
    assert _ws_choice(1, 0, 24, 3072, 4096) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 16, 6144, 16384) == "fewrows_m32_ws"
    assert _ws_choice(0, 0, 4, 6144, 16384) != "fewrows_m32_ws"
    assert _ws_choice(0, 0, 8, 3072, 2048) != "fewrows_m32_ws"      # K below 4096
    assert _ws_choice(0, 0, 1, 4096, 4096) == "skinny_m8_ws"        # 256 strips: a whole round
    assert _ws_choice(0, 0, 8, 9000, 8192) != "fewrows_m32_ws"      # past 8192 columns: no plan
    assert _ws_choice(0, 0, 24, 6144, 8192) == "mfma16_32x64x64_2x2_sched_splitk"   # 32-row tiles
    # 96 strips of 32 columns x 2 chunks; 96 strips of 64 columns x 2 chunks
    assert sg.sgemm_workspace_size(0, 0, 16, 3072, 8192, 1) == 4096 + 96 * 2 * 2 * 1024
    assert sg.sgemm_workspace_size(0, 0, 16, 6144, 4096, 1) == 4096 + 96 * 2 * 4 * 1024
    assert _ws_choice(0, 0, 8, 512, 8192) != "fewrows_m32_ws"       # too few strips for a long K
    assert _ws_choice(0, 0, 4, 1024, 65536) == "skinny_fixed_m8"    # beyond the measured K
    assert _ws_choice(0, 0, 8, 1024, 1024) == "fewrows_m32"         # K too short to split
    assert _ws_choice(0, 0, 32, 1024, 4096) != "fewrows_m32_ws"     # 32-row tiles fill C
    assert _ws_choice(0, 0, 24, 2048, 16384) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _ws_choice(0, 1, 16, 1024, 4096) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _ws_choice(0, 0, 8, 1024, 8192, ws_bytes=4096) == "fewrows_m32"   # workspace too small
    assert _ws_choice(0, 0, 8, 1024, 8192, batch=2) != "fewrows_m32_ws"
    # 64 strips x 4 chunks of 2048, one 16-row block of 256 floats per lane
    assert sg.sgemm_workspace_size(0, 0, 8, 1024, 8192, 1) == 4096 + 64 * 4 * 1024
    # 128 strips x 2 chunks, two 16-row blocks
    assert sg.sgemm_workspace_size(0, 0, 32, 2048, 4096, 1) == 4096 + 128 * 2 * 2 * 1024
    try:   # the split sums in a fixed order: allowed without atomics
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_NOT_ALLOWED) == sg.SGEMM_OK
        assert _ws_choice(0, 0, 8, 1024, 8192) == "fewrows_m32_ws"
    finally:
        sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED)
    # without a workspace, B transposed and up to 16 rows: the unsplit
    # few-rows kernel from 1024 columns at a K up to 2048
    assert _op_choice(0, 1, 8, 1024, 1024) == "fewrows_m32"
    assert _op_choice(0, 1, 16, 1024, 2048) == "fewrows_m32"
    assert _op_choice(0, 1, 8, 1024, 4096) == "mfma16_64x64x64_4x2_pipe_splitk"


def test_select_split_k_below_one_round(lib):
    """Fewer 64x64 tiles than CUs with a long K: K is split over workgroups
    ((64, 8192, 8192): 84 us split against 139 us on 128 tiles); from 32 to
    64 rows on the ordered loop's split tiles ((64, 8192, 8192) 111.5 against
    102.9 TFLOP/s, (48, 8192, 8192) 80.7 against 78.5, (64, 2048, 8192) 29.1
    against 31.9 us), above that the split 64x64 pipeline."""
    assert _op_choice(0, 0, 64, 8192, 8192) == "mfma16_64x64x64_4x2_sched_splitk"
    assert _op_choice(0, 0, 48, 8192, 8192) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 0, 64, 2048, 8192) == "mfma16_32x64x64_2x2_sched_splitk"
    assert _op_choice(0, 0, 128, 4096, 4096) == "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 0, 128, 4096, 1024) != "mfma16_64x64x64_4x2_pipe_splitk"
    assert _op_choice(0, 0, 1024, 1024, 1024) == "mfma16_64x64x64_4x2_sched"


def test_select_tile_fill_and_split_between_rounds(lib):
    """128-row tiles lose to 64x64 ones when much of them sticks out of C;
    between one and two 64x64 tiles per CU with a long K, K split on the
    ordered loop ((192, 8192, 8192): 121 vs 102 TFLOP/s on 128x64 tiles).
    One 64x64 tile per CU scores the split and unsplit forms within the
    model's error ((256, 4096, 4096): 115.7 unsplit, 113.1 split)."""
    assert _op_choice(0, 0, 192, 8192, 8192) == "mfma16_64x64x64_4x2_sched_splitk"
    assert _op_choice(0, 0, 192, 16384, 4096) == "mfma16_64x64x64_4x2_sched"
    assert _op_choice(0, 0, 448, 4096, 8192) == "mfma16_128x64x64_4x2_sched"
    assert _op_choice(0, 0, 256, 4096, 4096).startswith("mfma16_64x64x64_4x2_sched")


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = sg.sgemm_status_string(st)
        assert s and s != "unknown status"
    assert sg.sgemm_status_string(12345) == "unknown status"


def test_select_variant_is_pure(lib):
    # No launch, no HIP call: usable without a GPU.
    big = sg.sgemm_select_variant(4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE, 4096)
    assert sg.sgemm_variant_name(big).startswith("mfma32")
    tiny = sg.sgemm_select_variant(3, 5, 7, 1.0, FAKE, 7, FAKE, 5, 0.0, FAKE, 5)
    assert sg.sgemm_variant_name(tiny) == "simple"
    assert sg.sgemm_select_variant(0, 5, 7, 1.0, None, 7, None, 5, 0.0, None, 5) == sg.SGEMM_NO_KERNEL
    assert sg.sgemm_select_variant(3, 5, 7, 0.0, None, 7, None, 5, 0.5, FAKE, 5) == sg.SGEMM_NO_KERNEL
    assert sg.sgemm_select_variant(3, 5, 7, 1.0, FAKE, 6, FAKE, 5, 0.0, FAKE, 5) == sg.SGEMM_ERR_LD
    for shape in ((4095, 4097, 1023), (127, 129, 17), (1, 4096, 4096), (8192, 1024, 8192)):
        M, N, K = shape
        v = sg.sgemm_select_variant(M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N)
        assert 0 <= v < sg.sgemm_num_variants()


def test_ceiling_argument_checks(lib):
    assert sg.sgemm_ceiling_mfma(8, 1, 1, FAKE)[0] == -1
    assert sg.sgemm_ceiling_mfma(32, 0, 1, FAKE)[0] == -1
    assert sg.sgemm_ceiling_fma(1, 0, FAKE)[0] == -1
    assert sg.sgemm_ceiling_copy(FAKE, FAKE, 6, 1) == -1
    assert sg.sgemm_ceiling_copy(FAKE + 4, FAKE, 8, 1) == -1
    assert sg.sgemm_ceiling_read(FAKE, 6, 1, FAKE) == -1
    assert sg.sgemm_ceiling_read(FAKE + 4, 8, 1, FAKE) == -1
    assert sg.sgemm_ceiling_read(FAKE, 8, 0, FAKE) == -1
    assert sg.sgemm_ceiling_read(FAKE, 8, 1, None) == -1
    assert sg.sgemm_ceiling_empty(0) == -1


def test_no_device_is_reported_not_crashed(lib):
    """On a machine without a gfx950 GPU a valid call returns
    SGEMM_ERR_DEVICE (run in a child process; skipped when a GPU is present)."""
    code = (
        "import torch, sys\n"
        "if torch.cuda.is_available(): sys.exit(3)\n"
        "import dense_fp32_gemm_sgemm_amd as sg\n"
        "st = sg.sgemm(4, 4, 4, 1.0, 0x1000, 4, 0x1000, 4, 0.0, 0x1000, 4, 0)\n"
        "sys.exit(0 if st == sg.SGEMM_ERR_DEVICE else 1)\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    if res.returncode == 3:
        pytest.skip("a GPU is visible")
    assert res.returncode == 0, res.stdout + res.stderr


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIBRARY", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()


def _skinny_full_k(tb, N, K, batch):
    """The vector-unit few-rows kernel's one-pass form (no atomics): B not
    transposed, at least 64 strips of 32 columns over the batch, N*K <= 2^26."""
    return not tb and -(-N // 32) * batch >= 64 and N * K <= (1 << 26)


def test_atomics_mode_setting(lib):
    assert sg.sgemm_get_atomics_mode() == sg.SGEMM_ATOMICS_ALLOWED
    try:
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_NOT_ALLOWED) == sg.SGEMM_OK
        assert sg.sgemm_get_atomics_mode() == sg.SGEMM_ATOMICS_NOT_ALLOWED
        assert sg.sgemm_set_atomics_mode(7) == sg.SGEMM_ERR_OP
        assert sg.sgemm_get_atomics_mode() == sg.SGEMM_ATOMICS_NOT_ALLOWED
    finally:
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED) == sg.SGEMM_OK
    assert sg.sgemm_get_atomics_mode() == sg.SGEMM_ATOMICS_ALLOWED


def test_atomics_not_allowed_selection(lib):
    """With atomics not allowed the automatic choice takes no K-split variant
    and the vector-unit few-rows kernel only in its one-pass form, over a grid
    of shapes, orientations and batches that includes every case where the
    default choice splits; with atomics allowed again the choice is the
    default one."""
    dims = (1, 3, 8, 15, 24, 48, 64, 96, 127, 192, 320, 512, 1024, 4097)
    ks = (17, 100, 256, 1024, 4096, 16384, 100000)
    default, split_seen = {}, 0
    for ta in (0, 1):
        for tb in (0, 1):
            for batch in (1, 7):
                for M in dims:
                    for N in dims:
                        for K in ks:
                            if M * N * K * batch > 2 ** 37:
                                continue
                            name = _op_choice(ta, tb, M, N, K, batch)
                            default[(ta, tb, batch, M, N, K)] = name
                            split_seen += name.endswith("_splitk")
    assert split_seen > 100
    try:
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_NOT_ALLOWED) == sg.SGEMM_OK
        for (ta, tb, batch, M, N, K) in default:
            name = _op_choice(ta, tb, M, N, K, batch)
            assert not name.endswith("_splitk"), (ta, tb, batch, M, N, K, name)
            if name == "skinny_m8":
                assert _skinny_full_k(tb, N, K, batch), (ta, tb, batch, M, N, K)
    finally:
        sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED)
    for key, name in list(default.items())[::37]:
        assert _op_choice(key[0], key[1], key[3], key[4], key[5], key[2]) == name


def test_tile_choice_against_measured_rates(lib):
    """Every shape of the committed tile-family measurements
    (profiles/tile_choice_mi355x.md: every family timed on an MI355X as
    device time per call): the automatic choice of sgemm() is a measured
    family within 5% of the fastest family it may take (no split tail),
    and the choice with a workspace within 5% of the fastest of all --
    on every shape but at most two, which stay within 10%; the geometric
    mean of both is at least 0.98 of the fastest."""
    import math
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "tile_choice_mi355x.md")
    lines = open(path).read().splitlines()
    head = [h.strip() for h in next(l for l in lines if l.startswith("| M x N")).split("|")[1:-1]]
    fam = {"256x256": "mfma32_256x256x32_2x2_sched", "128x128 w4": "mfma16_128x128x32_2x2_sched",
           "128x128 w8": "mfma16_128x128x64_4x2_sched", "128x64": "mfma16_128x64x64_4x2_sched",
           "64x64": "mfma16_64x64x64_4x2_sched", "64x64 split-K": "mfma16_64x64x64_4x2_sched_splitk",
           "32x64": "mfma16_32x64x64_2x2_sched", "32x64 split-K": "mfma16_32x64x64_2x2_sched_splitk",
           "128x128 w4 tail": "mfma16_128x128x32_2x2_sched_tail",
           "128x128 w8 tail": "mfma16_128x128x64_4x2_sched_tail",
           "128x64 tail": "mfma16_128x64x64_4x2_sched_tail", "64x64 tail": "mfma16_64x64x64_4x2_sched_tail",
           "edge split": "edge_split"}
    ws_bytes = 4096 + (32 << 20)
    fracs, fracs_ws = [], []
    for line in lines:
        cells = [c.strip() for c in line.split("|")[1:-1]]
        if not cells or not cells[0][:1].isdigit():
            continue
        M, N, K = (int(x) for x in cells[0].split("x"))
        ta, tb = (1 if cells[1][0] == "T" else 0), (1 if cells[1][1] == "T" else 0)
        rates = {fam[h]: float(v.replace("*", "")) for h, v in zip(head, cells) if h in fam and v != "-"}
        plain = {k: v for k, v in rates.items() if not k.endswith("_tail")}
        name = _op_choice(ta, tb, M, N, K)
        assert name in plain, (cells[0], cells[1], name)
        fracs.append(plain[name] / max(plain.values()))
        v = sg.sgemm_strided_batched_ws_select_variant(ta, tb, M, N, K, 1.0, FAKE, M if ta else K, 0, FAKE,
                                                       K if tb else N, 0, 0.0, FAKE, N, 0, 1, ws_bytes)
        wname = sg.sgemm_variant_name(v)
        assert wname in rates, (cells[0], cells[1], wname)
        fracs_ws.append(rates[wname] / max(rates.values()))
    assert len(fracs) >= 80
    for f in (fracs, fracs_ws):
        assert min(f) >= 0.90 and sum(1 for x in f if x < 0.95) <= 2, sorted(f)[:4]
        assert math.exp(sum(math.log(x) for x in f) / len(f)) >= 0.98


def test_few_tiles_with_long_k_always_split(lib):
    """With few output tiles and a long K the automatic choice always spreads
    K over many workgroups: a K-split variant, or a streaming kernel whose
    waves split K (few rows, few columns, the vector-unit few-rows kernel),
    never a single-pass tile kernel with a handful of workgroups (tiny
    problems, at most 2^20 multiply-adds, excepted)."""
    streaming = {"fewrows_m32", "skinny_m8", "narrow_n16"}
    dims_m = (1, 8, 16, 17, 24, 31, 32, 33, 48, 64, 65, 96, 128, 200, 300)
    dims_n = (1, 15, 16, 17, 48, 63, 64, 65, 100, 128, 200, 300, 700, 1000)
    for ta in (0, 1):
        for tb in (0, 1):
            for M in dims_m:
                for N in dims_n:
                    for K in (1024, 2048, 8192, 65536):
                        for batch in (1, 3):
                            if M * N * K * batch <= (1 << 20):
                                continue  # launch-latency bound: one lane per output
                            if -(-M // 64) * -(-N // 64) * batch >= 64:
                                continue  # enough 64x64 tiles
                            name = _op_choice(ta, tb, M, N, K, batch)
                            assert name.endswith("_splitk") or name in streaming, (ta, tb, M, N, K, batch, name)


def test_select_fuzz_valid_and_stable(lib):
    """Random problems (every size class, orientation, batch and both atomics
    modes): the automatic choice is a valid variant, the same on a repeated
    call, and free of K-split variants when atomics are not allowed."""
    import random
    rnd = random.Random(1234)
    nv = sg.sgemm_num_variants()

    def dim():
        r = rnd.random()
        if r < 0.3:
            return rnd.choice((1, 2, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 255, 256, 257))
        if r < 0.8:
            return rnd.randint(1, 3000)
        return rnd.randint(3000, 70000)

    try:
        for i in range(6000):
            M, N, K = dim(), dim(), dim()
            batch = rnd.choice((1, 1, 1, 2, 7, 100))
            if M * N * K * batch > 2 ** 44:
                continue
            ta, tb = rnd.randint(0, 1), rnd.randint(0, 1)
            mode = sg.SGEMM_ATOMICS_ALLOWED if i % 3 else sg.SGEMM_ATOMICS_NOT_ALLOWED
            assert sg.sgemm_set_atomics_mode(mode) == sg.SGEMM_OK
            v = sg.sgemm_strided_batched_select_variant(
                ta, tb, M, N, K, 1.0, FAKE, M if ta else K, M * K, FAKE, K if tb else N, K * N, 0.0,
                FAKE, N, M * N, batch)
            assert 0 <= v < nv, (ta, tb, M, N, K, batch, v)
            again = sg.sgemm_strided_batched_select_variant(
                ta, tb, M, N, K, 1.0, FAKE, M if ta else K, M * K, FAKE, K if tb else N, K * N, 0.0,
                FAKE, N, M * N, batch)
            assert again == v
            if mode == sg.SGEMM_ATOMICS_NOT_ALLOWED:
                assert not sg.sgemm_variant_name(v).endswith("_splitk"), (ta, tb, M, N, K, batch)
    finally:
        sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED)


# ---------------------------------------------------------------- launch planning

def _no_gpu():
    import torch
    return not torch.cuda.is_available()


def test_scale_any_width_is_not_a_grid_error(lib):
    """alpha = 0 (or K = 0) scales C by beta with a grid-stride kernel, so a C
    wider than 65535 blocks of 64 columns is valid: the call gets past the
    launch plan to the device check (no GPU here: SGEMM_ERR_DEVICE)."""
    if not _no_gpu():
        pytest.skip("a GPU is present")
    N = 5_000_000
    assert sg.sgemm(1, N, 0, 1.0, None, 1, None, N, 0.5, FAKE, N, 0) == sg.SGEMM_ERR_DEVICE
    assert sg.sgemm(3, N, 7, 0.0, None, 7, None, N, 2.0, FAKE, N, 0) == sg.SGEMM_ERR_DEVICE
    # the one-lane kernel strides too: forced on a very wide problem
    simple = sg.variant_names().index("simple")
    assert sg.sgemm_ex(1, N, 4, 1.0, FAKE, 4, FAKE, N, 0.0, FAKE, N, 0, simple) == sg.SGEMM_ERR_DEVICE


def test_grid_too_large_is_reported_before_any_launch(lib):
    """A problem whose tile grid exceeds the HIP limits (2^32 work-items along
    x) returns SGEMM_ERR_GRID from the launch plan, before the device is
    touched -- for the automatic choice, a forced variant, the choice query,
    and a batch split into several chunks of 65535 slices."""
    M = N = 1 << 20
    st = sg.sgemm(M, N, 1024, 1.0, FAKE, 1024, FAKE, N, 0.0, FAKE, N, 0)
    assert st == sg.SGEMM_ERR_GRID, st
    assert sg.sgemm_select_variant(M, N, 1024, 1.0, FAKE, 1024, FAKE, N, 0.0, FAKE, N) == sg.SGEMM_ERR_GRID
    v = sg.variant_names().index("mfma16_64x64x16_2x2")
    assert sg.sgemm_ex(M, N, 64, 1.0, FAKE, 64, FAKE, N, 0.0, FAKE, N, 0, v) == sg.SGEMM_ERR_GRID
    # 70000 slices: two chunks, each with the same oversized grid
    Mb, Nb = 1 << 19, 1 << 19
    args = (0, 0, Mb, Nb, 64, 1.0, FAKE, 64, 0, FAKE, Nb, 0, 0.0, FAKE, Nb, Mb * Nb, 70000)
    assert sg.sgemm_strided_batched_ex(*args, 0, v) == sg.SGEMM_ERR_GRID
    assert "nothing was enqueued" in sg.sgemm_status_string(sg.SGEMM_ERR_GRID)


def test_large_batch_within_limits_passes_the_plan(lib):
    """Just inside the limits the plan passes (no GPU here: the device check
    answers)."""
    if not _no_gpu():
        pytest.skip("a GPU is present")
    args = (0, 0, 64, 64, 64, 1.0, FAKE, 64, 4096, FAKE, 64, 4096, 0.0, FAKE, 64, 4096, 200000)
    assert sg.sgemm_strided_batched(*args, 0) == sg.SGEMM_ERR_DEVICE


@pytest.mark.parametrize("which", ["A", "B", "C"])
def test_strided_one_row_view_is_rejected(which):
    """A one-row view whose elements are not adjacent (column stride != 1) is
    not a row-major matrix: the binding refuses it instead of reading or
    writing its row as if it were packed."""
    import torch
    base = torch.zeros(4, 512)
    strided = base[:1, ::8]                      # shape (1, 64), strides (512, 8)
    assert strided.shape == (1, 64) and strided.stride() == (512, 8)
    A = torch.zeros(1, 64) if which != "A" else strided
    B = torch.zeros(64, 64)
    C = torch.zeros(1, 64) if which != "C" else strided
    if which == "B":
        B = torch.zeros(1, 512)[:, ::8]          # K = 1 row of B, strided
        A = torch.zeros(1, 1)
    with pytest.raises(ValueError, match="row-major"):
        sg.gemm(A, B, C)


def test_edge_split_only_where_the_benchmark_times_it(lib):
    """The tile-choice benchmark times the edge split only where a thin edge
    exists (bench.has_thin_edge); the automatic choice must never take it
    anywhere else, or its tables would miss the chosen form.  Seeded shapes
    around tile boundaries, every orientation."""
    import random
    import bench
    rng = random.Random(7)
    seen = 0
    for _ in range(400):
        M = rng.choice((32, 64, 128, 256)) * rng.randint(2, 40) + rng.randint(-40, 40)
        N = rng.choice((64, 128, 256)) * rng.randint(2, 40) + rng.randint(-40, 40)
        K = rng.choice((257, 999, 1000, 1023, 2048, 4097))
        ta, tb = rng.randint(0, 1), rng.randint(0, 1)
        if _op_choice(ta, tb, M, N, K) == "edge_split":
            seen += 1
            assert bench.has_thin_edge(M, N, K), (ta, tb, M, N, K)
    assert seen >= 20, seen
