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


def _write_trace(path, rows, counters=False):
    import csv
    keys = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
            "Grid_Size_X"] + (["Counter_Name", "Counter_Value"] if counters else [])
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_summary_splits_jobs_by_separators(tmp_path):
    """Kernel-only time per call: the dispatches between a job's graph-phase
    separator and its end separator, divided by the calls the log names."""
    rows, t, d = [], 0, 0

    def disp(name, dur, grid=256, wg=256):
        nonlocal t, d
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Start_Timestamp": t,
                     "End_Timestamp": t + dur, "Workgroup_Size_X": wg, "Grid_Size_X": grid})
        t += dur + 100
        d += 1

    sep = "sg950::empty_kernel()"
    for job, dur, n_calls in ((0, 1000, 6), (1, 3000, 4)):
        disp(sep, 10, grid=64 * bench.mark_code(job, 0), wg=64)
        disp("void sg950::sched_kernel<...>(sg950::Problem)", 99999)   # eager phase: not counted
        disp(sep, 10, grid=64 * bench.mark_code(job, 1), wg=64)
        for _ in range(n_calls):
            disp("void sg950::scale_kernel(int)", 200)
            disp("void sg950::sched_kernel<...>(sg950::Problem)", dur)
        disp(sep, 10, grid=64 * bench.mark_code(job, 2), wg=64)
    tr = tmp_path / "kt.csv"
    _write_trace(tr, rows)
    log = tmp_path / "run.log"
    with open(log, "w") as f:
        f.write("not json\n")
        f.write(json.dumps({"job": 0, "M": 64, "N": 64, "K": 64, "variant": "a", "graph_reps": 3,
                            "graph_replays": 2, "us_device": 1.5, "us_launch": 7.0}) + "\n")
        f.write(json.dumps({"job": 1, "M": 128, "N": 64, "K": 64, "variant": "b", "graph_reps": 2,
                            "graph_replays": 2, "us_device": 3.5, "us_launch": 9.0}) + "\n")
    table = bench.trace_summary(str(tr), str(log)).strip().splitlines()
    assert len(table) == 4
    r0 = [c.strip() for c in table[2].split("|")[1:-1]]
    r1 = [c.strip() for c in table[3].split("|")[1:-1]]
    assert r0[:4] == ["0", "64x64x64", "NN", "a"] and r0[4] == "2.00" and r0[5] == "1.20"
    assert r1[4] == "2.00" and r1[5] == "3.20"


def test_counter_summary_means_per_job(tmp_path):
    rows = []
    sep = "sg950::empty_kernel()"
    did = 0
    for job, vals in ((0, (10.0, 30.0)), (1, (5.0,))):
        rows.append({"Dispatch_Id": did, "Kernel_Name": sep, "Start_Timestamp": 0, "End_Timestamp": 1,
                     "Workgroup_Size_X": 64, "Grid_Size_X": 64 * bench.mark_code(job, 1),
                     "Counter_Name": "X", "Counter_Value": 0})
        did += 1
        for v in vals:
            rows.append({"Dispatch_Id": did, "Kernel_Name": "void sg950::scale_kernel(int)",
                         "Start_Timestamp": 0, "End_Timestamp": 1, "Workgroup_Size_X": 256,
                         "Grid_Size_X": 256, "Counter_Name": "X", "Counter_Value": 1e9})
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": "void sg950::sched_kernel<1>()",
                         "Start_Timestamp": 0, "End_Timestamp": 1, "Workgroup_Size_X": 256,
                         "Grid_Size_X": 256, "Counter_Name": "X", "Counter_Value": v})
            did += 1
        rows.append({"Dispatch_Id": did, "Kernel_Name": sep, "Start_Timestamp": 0, "End_Timestamp": 1,
                     "Workgroup_Size_X": 64, "Grid_Size_X": 64 * bench.mark_code(job, 2),
                     "Counter_Name": "X", "Counter_Value": 0})
        did += 1
    # job 2: two calls of two kernels each (the edge split): summed per call
    rows.append({"Dispatch_Id": did, "Kernel_Name": sep, "Start_Timestamp": 0, "End_Timestamp": 1,
                 "Workgroup_Size_X": 64, "Grid_Size_X": 64 * bench.mark_code(2, 1),
                 "Counter_Name": "X", "Counter_Value": 0})
    did += 1
    for v in (10.0, 1.0, 12.0, 1.0):
        rows.append({"Dispatch_Id": did, "Kernel_Name": "void sg950::sched_kernel<1>()" if v > 1 else
                     "void sg950::narrow_kernel<false>()", "Start_Timestamp": 0, "End_Timestamp": 1,
                     "Workgroup_Size_X": 256, "Grid_Size_X": 256, "Counter_Name": "X", "Counter_Value": v})
        did += 1
    rows.append({"Dispatch_Id": did, "Kernel_Name": sep, "Start_Timestamp": 0, "End_Timestamp": 1,
                 "Workgroup_Size_X": 64, "Grid_Size_X": 64 * bench.mark_code(2, 2),
                 "Counter_Name": "X", "Counter_Value": 0})
    p = tmp_path / "cc.csv"
    _write_trace(p, rows, counters=True)
    log = tmp_path / "run.log"
    log.write_text(json.dumps({"job": 0, "M": 1, "N": 2, "K": 3, "variant": "v"}) + "\n" +
                   json.dumps({"job": 2, "M": 4, "N": 5, "K": 6, "variant": "edge_split", "steps": 2}) + "\n")
    out = bench.counter_summary(str(p), str(log))
    assert [o["job"] for o in out] == [0, 1, 2]
    assert out[0]["counters"]["X"] == 20.0 and out[0]["dispatches"] == 2 and out[0]["M"] == 1
    assert out[1]["counters"]["X"] == 5.0
    assert out[2]["counters"]["X"] == 12.0 and out[2]["dispatches"] == 4 and out[2]["calls"] == 2
    assert len(out[2]["kernels"]) == 2


def _jsonl(path, recs):
    path.write_text("".join(json.dumps(r) + "\n" for r in recs))
    return str(path)


def test_sweep_md_binding_roof_and_vendor_ratio(tmp_path):
    """The sweep table keeps each record's roof, its fraction, the cold read
    floor and vendor / ours; the workspace run's columns join by shape."""
    ceil = {"mode": "ceilings", "mfma_f32_32x32x2_tflops": 155.0, "mfma_f32_16x16x4_tflops": 141.0,
            "valu_fma_f32_tflops": 128.0, "hbm_copy_gbs": 4500.0, "hbm_read_gbs": 5900.0,
            "dispatch_floor_us": 1.5}
    rec = {"mode": "sweep", "M": 1, "N": 4096, "K": 4096, "variant": "skinny_m8", "us_device": 12.0,
           "tflops_device": 2.8, "us_launch": 14.0, "us_cold": 20.0, "bound": "hbm", "rated_on": "us_cold",
           "floor_us": {"mfma": 0.2, "hbm": 11.4, "latency": 1.5}, "frac_of_bound": 0.57,
           "frac_datasheet": 0.011, "us_read_cold": 11.6, "torch_mm_us_device": 18.0}
    ws = dict(rec, variant="skinny_m8_ws", us_device=13.0, us_cold=15.0)
    md = bench.sweep_md(_jsonl(tmp_path / "s.jsonl", [ceil, rec]), _jsonl(tmp_path / "w.jsonl", [ws]))
    row = [l for l in md.splitlines() if l.startswith("| 1x4096x4096")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[6] == "hbm (cold)" and cells[8] == "0.570" and cells[10] == "11.60"
    assert cells[12] == "1.50"                       # vendor 18 / ours 12
    assert cells[13:] == ["skinny_m8_ws", "13.00", "2.80", "15.00"]


def test_few_rows_md_ratio_uses_the_better_choice(tmp_path):
    rec = {"mode": "few-rows", "M": 1, "N": 4096, "K": 4096, "ops": "NN", "auto": "skinny_m8",
           "auto_ws": "skinny_m8_ws", "us_device_auto": 12.0, "us_device_auto_ws": 10.0,
           "us_cold_auto": 20.0, "auto_gbs_cold": 3355.0, "us_device_skinny_m8": 12.0,
           "us_device_mfma16_64x64x64_4x2_pipe_splitk": 23.0, "us_device_fewrows_m32": 15.0,
           "torch_mm_us_device": 15.0}
    md = bench.few_rows_md(_jsonl(tmp_path / "f.jsonl", [rec]))
    row = [l for l in md.splitlines() if l.startswith("| 1x4096x4096")][0]
    assert row.rstrip().endswith("| 15.00 | 1.50 |")   # vendor 15 / min(12, 10)
    assert "geometric mean 1.500 over 1 shapes" in md


def test_variants_md_marks_best_forced_and_auto_ratio(tmp_path):
    recs = [{"M": 64, "N": 64, "K": 64, "variant": "a", "forced": True, "us_device": 2.0, "tflops_device": 1.0},
            {"M": 64, "N": 64, "K": 64, "variant": "b", "forced": True, "us_device": 1.0, "tflops_device": 2.0},
            {"M": 64, "N": 64, "K": 64, "variant": "b", "forced": False, "us_device": 1.0,
             "tflops_device": 1.9}]
    md = bench.variants_md([_jsonl(tmp_path / "v.jsonl", recs)])
    row = [l for l in md.splitlines() if l.startswith("| 64x64x64")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2:] == ["1.00", "**2.00**", "b", "1.90", "0.950"]


def test_counters_md_busy_fetch_and_hit_rate(tmp_path):
    """MFMA busy from the deterministic busy count (2MNK / 64 per SIMD), fetch
    scaled by the copy calibration, L2 hit rate and LDS conflict share."""
    M = N = K = 1024
    busy = 2.0 * M * N * K / 64                     # summed over the 1024 SIMDs
    base = {"job": 0, "M": M, "N": N, "K": K, "variant": "v", "dispatches": 1}
    passes = [dict(base, counters={"SQ_VALU_MFMA_BUSY_CYCLES": busy, "GRBM_GUI_ACTIVE": 8 * 40000.0,
                                   "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 100.0}),
              dict(base, counters={"FETCH_SIZE": 1000.0}), dict(base, counters={"WRITE_SIZE": 4096.0}),
              dict(base, counters={"TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0})]
    paths = []
    for i, p in enumerate(passes):
        f = tmp_path / ("p%d.json" % i)
        f.write_text(json.dumps([p]))
        paths.append(str(f))
    times = _jsonl(tmp_path / "t.jsonl", [{"M": M, "N": N, "K": K, "variant": "v", "us_device": 20.0}])
    md = bench.counters_md(paths, times)
    row = [l for l in md.splitlines() if l.startswith("| 1024x1024x1024")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    ideal = busy / 1024                             # 32768 cycles
    assert cells[2] == "%.1f%%" % (100 * ideal / 40000.0)
    assert cells[3] == "20.00" and cells[4] == "%.1f%%" % (100 * ideal / (20.0 * 1e3 * 2.38))
    assert cells[5] == "2.0"                        # 1000 KiB x 1024 x 2.0 / 1e6
    assert cells[10] == "75.0%" and cells[11] == "10.0%"
