"""GPU parity of the fixed-order split of the last round of tiles (the
``*_sched_tail`` variants and the workspace entry points), through the C ABI
against the fp64 oracle.

The split form writes partial tiles to a workspace and the workgroup that
finishes a tile's K ranges last adds them in range order, so besides the
oracle's bars (exact on integer data, 1e-5 normalized error on real data)
every call must be bitwise repeatable and must leave the workspace's
counters at zero for the next call."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import dense_fp32_gemm_sgemm_amd as sg  # noqa: E402
from tests.gpu_util import DevMatrix, run  # noqa: E402
from workloads import draw, draw_workload, ragged_workloads, sweep_workloads  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-5
WS_BYTES = 4096 + (32 << 20)   # the largest workspace any problem can use
VN = sg.variant_names()

# (variant, shape): each shape gives the family a last, partial round of
# tiles; the first of each pair also has whole rounds before it (the
# whole-tile and split workgroups share one grid), and K is ragged where the
# family's slab depth does not divide it.
CASES = [
    ("mfma16_128x128x32_2x2_sched_tail", (2944, 2944, 1000)),
    ("mfma16_128x128x32_2x2_sched_tail", (300, 520, 1000)),
    ("mfma16_128x128x64_4x2_sched_tail", (2100, 2100, 1500)),
    ("mfma16_128x128x64_4x2_sched_tail", (400, 300, 2000)),
    ("mfma16_128x64x64_4x2_sched_tail", (1000, 1000, 2048)),
    ("mfma16_128x64x64_4x2_sched_tail", (1500, 2200, 700)),
    ("mfma16_64x64x64_4x2_sched_tail", (600, 700, 3000)),
    ("mfma16_64x64x64_4x2_sched_tail", (1500, 1400, 1100)),
]


def say(*a):
    print(*a, flush=True)


def new_ws():
    return torch.zeros(WS_BYTES, dtype=torch.uint8, device="cuda")


def counters_zero(ws):
    return bool((ws[:4096] == 0).all().item())


def _ids(c):
    return "%s-%dx%dx%d" % ((c[0],) + c[1])


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_tail_form_against_oracle(case):
    name, (M, N, K) = case
    v = VN.index(name)
    ws = new_ws()
    say("tail", name, (M, N, K))
    A, B, _ = draw(M, N, K, seed=M + N + K)
    C1 = run(A, B, variant=v, workspace=ws)
    assert counters_zero(ws), "counters left set"
    ref, den = oracle.gemm(A, B)
    err = oracle.normalized_error(C1, ref, den)
    assert err <= TOL, "%s %s: normalized error %.3g" % (name, (M, N, K), err)
    C2 = run(A, B, variant=v, workspace=ws)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "not bitwise repeatable"
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K + 1, kind="int", with_c=True)
    C3 = run(Ai, Bi, Ci, 1.0, 1.0, variant=v, workspace=ws)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    assert oracle.exact_match(C3, ref), "%s %s: integer result differs" % (name, (M, N, K))
    assert counters_zero(ws)


@pytest.mark.parametrize("ops", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
@pytest.mark.parametrize("name", ["mfma16_128x128x32_2x2_sched_tail", "mfma16_128x128x64_4x2_sched_tail"])
def test_tail_form_transposed(name, ops):
    ta, tb = ops
    M, N, K = 400, 520, 1000
    v = VN.index(name)
    ws = new_ws()
    A, B, Cin = draw(M, N, K, seed=77, with_c=True)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    say("tail transposed", name, ops)
    C = run(As, Bs, Cin, 1.5, 0.5, variant=v, workspace=ws, trans_a=ta, trans_b=tb)
    ref, den = oracle.gemm(A, B, Cin, 1.5, 0.5)
    assert oracle.normalized_error(C, ref, den) <= TOL
    assert counters_zero(ws)


def test_tail_form_padded_misaligned_and_nan_c():
    """Odd leading dimensions, 4-byte (not 16-byte) aligned operands and a
    NaN-filled C with beta = 0; nothing outside C is written."""
    M, N, K = 700, 650, 1030
    v = VN.index("mfma16_128x128x32_2x2_sched_tail")
    ws = new_ws()
    A, B, _ = draw(M, N, K, seed=5)
    say("tail padded")
    C = run(A, B, None, 1.0, 0.0, variant=v, lds=(K + 3, N + 1, N + 5), offsets=(1, 3, 2),
            check_outside=True, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C, ref, den) <= TOL
    assert counters_zero(ws)


def test_workspace_reused_across_shapes_and_too_small():
    """One workspace serves calls of different shapes in turn; a workspace
    too small for the split runs the family's whole-tile loop (still
    correct); a misaligned one is an error."""
    ws = new_ws()
    v = VN.index("mfma16_128x128x32_2x2_sched_tail")
    for i, (M, N, K) in enumerate([(300, 520, 1000), (1024, 1024, 1024), (200, 900, 4000),
                                   (300, 520, 1000)]):
        Ai, Bi, _ = draw(M, N, K, seed=300 + i, kind="int")
        say("reuse", (M, N, K))
        C = run(Ai, Bi, variant=v, workspace=ws)
        ref, _ = oracle.gemm(Ai, Bi)
        assert oracle.exact_match(C, ref), (M, N, K)
        assert counters_zero(ws)
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    Ai, Bi, _ = draw(300, 520, 1000, seed=9, kind="int")
    C = run(Ai, Bi, variant=v, workspace=small)
    ref, _ = oracle.gemm(Ai, Bi)
    assert oracle.exact_match(C, ref)
    dA = torch.from_numpy(Ai).cuda()
    dB = torch.from_numpy(Bi).cuda()
    dC = torch.zeros(300, 520, device="cuda")
    st = sg.sgemm_strided_batched_ws(0, 0, 300, 520, 1000, 1.0, dA.data_ptr(), 1000, 0, dB.data_ptr(),
                                     520, 0, 0.0, dC.data_ptr(), 520, 0, 1, ws.data_ptr() + 4,
                                     WS_BYTES - 4, 0)
    assert st == sg.SGEMM_ERR_WORKSPACE


def test_automatic_choice_with_workspace():
    """The automatic choice of the workspace entry point takes the tail form
    where the last round is partial and no thin edge can be split off --
    3000^3 -- and the edge split at (4095, 4097, 1023), whose 4097 columns
    overrun the tiles by one; results meet the oracle (every element),
    integer copies exactly; 1024^3 through the same entry point likewise,
    whatever it chooses."""
    shapes = [(3000, 3000, 3000, 31)]
    shapes += [(w.M, w.N, w.K, w.seed) for w in ragged_workloads() if w.M == 4095]
    shapes += [(w.M, w.N, w.K, w.seed) for w in sweep_workloads() if w.M == 1024]
    for M, N, K, seed in shapes:
        need = sg.sgemm_workspace_size(0, 0, M, N, K, 1)
        v = sg.sgemm_strided_batched_ws_select_variant(0, 0, M, N, K, 1.0, 256, K, 0, 256, N, 0, 0.0,
                                                       256, N, 0, 1, WS_BYTES)
        say("auto ws", (M, N, K), sg.sgemm_variant_name(v), need)
        assert need <= WS_BYTES
        if M == 3000:
            assert sg.sgemm_variant_name(v).endswith("_tail") and need > 4096
        if M == 4095:
            assert sg.sgemm_variant_name(v) == "edge_split"
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
        A, B, _ = draw(M, N, K, seed=seed)
        C = run(A, B, workspace=ws)
        ref, den = oracle.gemm(A, B)
        assert oracle.normalized_error(C, ref, den) <= TOL
        Ai, Bi, _ = draw(M, N, K, seed=seed, kind="int")
        C = run(Ai, Bi, workspace=ws)
        ref, _ = oracle.gemm(Ai, Bi)
        assert oracle.exact_match(C, ref)
        assert counters_zero(ws)


def test_tail_form_in_a_graph():
    """A workspace call captured in a HIP graph replays exactly several
    times, with eager work between the replays (the counters are reset by
    each replay's own kernels)."""
    M, N, K = 1024, 1024, 1024
    Ai, Bi, Ci = draw(M, N, K, seed=11, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bi, Ci))
    out = torch.empty_like(dC0)
    ws = new_ws()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, workspace=ws)
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), "replay %d" % i
        assert counters_zero(ws)


def test_full_size_ragged_shape_with_workspace():
    """(4095, 4097, 1023) with B and C rows not 16-byte aligned, through the
    workspace entry point's automatic choice (the launch configuration the
    sweep times with a workspace): every element against the oracle."""
    w = [w for w in ragged_workloads() if w.M == 4095][0]
    A, B, _ = draw_workload(w)
    ws = new_ws()
    C = run(A, B, workspace=ws)
    ref, den = oracle.gemm(A, B)
    err = oracle.normalized_error(C, ref, den)
    say("4095x4097x1023 ws normalized error %.3g" % err)
    assert err <= TOL
