"""CPU tests: the benchmark's flop/byte accounting against figures the pages
print (tests/golden/page_figures.json, each entry with its source)."""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")
FIG = json.load(open(GOLDEN))


def close(x, want, rel):
    return abs(x - want) <= rel * abs(want) + 1e-12


def test_flops_4096():
    f = FIG["gemm_4096_gflop"]
    assert close(bench.flops(4096, 4096, 4096) / 1e9, f["value"], f["rel_tol"])


def test_bytes_and_intensity_4096():
    four = FIG["gemm_4096_four_matrix_mb"]
    assert close(bench.min_bytes(4096, 4096, 4096, beta=0.5) / 1e6, four["value"], four["rel_tol"])
    three = FIG["gemm_4096_three_matrix_mb"]
    assert close(bench.min_bytes(4096, 4096, 4096, beta=0.0) / 1e6, three["value"], three["rel_tol"])
    ai = FIG["gemm_4096_ai_accumulate"]
    assert close(bench.arithmetic_intensity(4096, 4096, 4096, beta=0.5), ai["value"], ai["rel_tol"])
    ai3 = FIG["gemm_4096_ai_three_matrix"]
    assert close(bench.arithmetic_intensity(4096, 4096, 4096, beta=0.0), ai3["value"], ai3["rel_tol"])


def test_naive_intensity():
    # one multiply-add (2 FLOP) per float of A and float of B (8 bytes)
    assert bench.flops(1, 1, 1) / 8.0 == FIG["naive_kernel_ai"]["value"]


def test_register_tile_reuse():
    r = FIG["lds_reads_per_fma"]
    assert bench.lds_reads_per_fma(1, 1) == r["tile_1x1"]
    assert bench.lds_reads_per_fma(8, 1) == r["tile_8x1"]
    assert bench.lds_reads_per_fma(8, 8) == r["tile_8x8"]


def test_tiled_global_traffic():
    g = FIG["global_load_gib_4096"]
    assert bench.tile_global_bytes(4096, 4096, 4096, 32, 32) / 2 ** 30 == g["tile_32"]
    assert bench.tile_global_bytes(4096, 4096, 4096, 128, 128) / 2 ** 30 == g["tile_128"]


@pytest.mark.parametrize("run", FIG["timed_runs"], ids=lambda r: str(r["ms"]))
def test_printed_rates_rederive(run):
    n = run["n"]
    gflops = bench.flops(n, n, n) / (run["ms"] * 1e-3) / 1e9
    assert close(gflops, run["gflops"], 5e-4), (gflops, run)


def test_bench_refuses_multi_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16
