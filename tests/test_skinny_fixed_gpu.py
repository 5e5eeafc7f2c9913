"""GPU parity of the fixed-order split few-rows form (``skinny_fixed_m8``
with a workspace) through the C ABI against the fp64 oracle.

The form splits B into (256-column strip, K chunk) workgroups; each chunk's
partial strip goes to the workspace and the strip's last chunk adds them in
chunk order.  Besides the oracle's bars (exact on integer data, 1e-5
normalized error on real data) every call must be bitwise repeatable and
leave the workspace's counters at zero."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import dense_fp32_gemm_sgemm_amd as sg  # noqa: E402
from tests.gpu_util import run  # noqa: E402
from workloads import draw  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-5
WS_BYTES = 4096 + (32 << 20)
V = sg.variant_names().index("skinny_fixed_m8")

# rows 1..8 (each register-block width), ragged N (not a multiple of the
# 256-column strip, nor of 4), K from one row to several chunks with a
# ragged last chunk
SHAPES = [
    (1, 4096, 4096), (2, 4096, 4096), (3, 1000, 3000), (4, 4097, 1023), (5, 2048, 4099),
    (8, 300, 7000), (1, 1, 1), (1, 3, 5), (2, 256, 1), (7, 4100, 129), (1, 16384, 700),
    (4, 512, 20000),
]


def say(*a):
    print(*a, flush=True)


def new_ws():
    return torch.zeros(WS_BYTES, dtype=torch.uint8, device="cuda")


def counters_zero(ws):
    return bool((ws[:4096] == 0).all().item())


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_fixed_form_against_oracle(shape):
    M, N, K = shape
    ws = new_ws()
    say("fixed few-rows", shape)
    A, B, _ = draw(M, N, K, seed=M * 7 + N + K)
    C1 = run(A, B, variant=V, workspace=ws)
    assert counters_zero(ws), "counters left set"
    ref, den = oracle.gemm(A, B)
    err = oracle.normalized_error(C1, ref, den)
    assert err <= TOL, "%s: normalized error %.3g" % (shape, err)
    C2 = run(A, B, variant=V, workspace=ws)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "not bitwise repeatable"
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K + 1, kind="int", with_c=True)
    C3 = run(Ai, Bi, Ci, 1.0, 1.0, variant=V, workspace=ws)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    assert oracle.exact_match(C3, ref), "%s: integer result differs" % (shape,)
    assert counters_zero(ws)


@pytest.mark.parametrize("trans_a", [False, True], ids=["NN", "TN"])
def test_fixed_form_alpha_beta_and_transposed_a(trans_a):
    M, N, K = 6, 1500, 2500
    ws = new_ws()
    A, B, Cin = draw(M, N, K, seed=41, with_c=True)
    As = np.ascontiguousarray(A.T) if trans_a else A
    say("fixed few-rows alpha/beta", trans_a)
    C = run(As, B, Cin, -1.25, 0.75, variant=V, workspace=ws, trans_a=trans_a)
    ref, den = oracle.gemm(A, B, Cin, -1.25, 0.75)
    assert oracle.normalized_error(C, ref, den) <= TOL
    assert counters_zero(ws)


@pytest.mark.parametrize("N", [777, 776])
def test_fixed_form_padded_misaligned_and_nan_c(N):
    """Odd leading dimensions and 4-byte aligned operands with a NaN-filled C
    and beta = 0 (N = 777: B read element by element; N = 776: as 16-byte
    vectors off 16-byte boundaries); nothing outside C written."""
    M, K = 3, 1234
    ws = new_ws()
    A, B, _ = draw(M, N, K, seed=8)
    say("fixed few-rows padded", N)
    C = run(A, B, None, 1.0, 0.0, variant=V, lds=(K + 3, N + 1, N + 5), offsets=(1, 3, 2),
            check_outside=True, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C, ref, den) <= TOL
    assert counters_zero(ws)


def test_fixed_form_without_or_with_small_workspace():
    """No workspace, or one too small for the partial strips: the few-rows
    kernel's other forms run instead (still within the bars); taller
    problems run as row blocks of 8."""
    for M, N, K, ws in [(2, 4096, 4096, None), (2, 4096, 4096, torch.zeros(64, dtype=torch.uint8, device="cuda")),
                        (19, 1000, 2000, None), (19, 1000, 2000, new_ws())]:
        Ai, Bi, _ = draw(M, N, K, seed=M + 3, kind="int")
        say("fixed few-rows fallback", (M, N, K), None if ws is None else ws.numel())
        C = run(Ai, Bi, variant=V, workspace=ws)
        ref, _ = oracle.gemm(Ai, Bi)
        assert oracle.exact_match(C, ref), (M, N, K)


def test_fixed_form_in_a_graph():
    """Captured in a HIP graph it replays exactly, with eager work between
    the replays (each replay's last chunks reset the counters)."""
    M, N, K = 4, 4096, 4096
    Ai, Bi, Ci = draw(M, N, K, seed=12, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bi, Ci))
    out = torch.empty_like(dC0)
    ws = new_ws()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=V, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=V, workspace=ws)
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), "replay %d" % i
        assert counters_zero(ws)


@pytest.mark.parametrize("shape", [(1, 512, 32768), (4, 1024, 65536), (1, 65536, 2048), (8, 5000, 16384)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_automatic_choice_with_workspace_takes_fixed_form(shape):
    """Through the workspace entry point's automatic choice these shapes
    take the fixed-order form (the workspace size the library reports is
    enough for it); results meet the oracle and repeat bit for bit."""
    M, N, K = shape
    need = sg.sgemm_workspace_size(0, 0, M, N, K, 1)
    v = sg.sgemm_strided_batched_ws_select_variant(0, 0, M, N, K, 1.0, 256, K, 0, 256, N, 0, 0.0, 256, N, 0, 1,
                                                   WS_BYTES)
    say("auto fixed few-rows", shape, sg.sgemm_variant_name(v), need)
    assert v == V and 4096 < need <= WS_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    A, B, _ = draw(M, N, K, seed=N + K)
    C1 = run(A, B, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C1, ref, den) <= TOL
    C2 = run(A, B, workspace=ws)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    Ai, Bi, _ = draw(M, N, K, seed=N + K + 1, kind="int")
    C3 = run(Ai, Bi, workspace=ws)
    ref, _ = oracle.gemm(Ai, Bi)
    assert oracle.exact_match(C3, ref)
    assert counters_zero(ws)


# The full-K strip kernel split over K through the workspace (skinny_m8_ws):
# strip counts from 64 to 255 (two to four ranges), ragged N (a partial last
# strip, N not a multiple of 4: element loads), ragged last range, M 1..8.
VWS = sg.variant_names().index("skinny_m8_ws")
WS_SPLIT_SHAPES = [(1, 4096, 4096), (2, 2048, 2048), (4, 4096, 4096), (8, 4096, 2048), (3, 4000, 3000),
                   (1, 2050, 4099), (6, 8000, 4096)]


@pytest.mark.parametrize("shape", WS_SPLIT_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_split_full_k_against_oracle(shape):
    M, N, K = shape
    ws = new_ws()
    say("split full-K few-rows", shape)
    A, B, _ = draw(M, N, K, seed=M * 5 + N + K)
    C1 = run(A, B, variant=VWS, workspace=ws)
    assert counters_zero(ws), "counters left set"
    ref, den = oracle.gemm(A, B)
    err = oracle.normalized_error(C1, ref, den)
    assert err <= TOL, "%s: normalized error %.3g" % (shape, err)
    C2 = run(A, B, variant=VWS, workspace=ws)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "not bitwise repeatable"
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K + 2, kind="int", with_c=True)
    C3 = run(Ai, Bi, Ci, 1.0, 1.0, variant=VWS, workspace=ws)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    assert oracle.exact_match(C3, ref), "%s: integer result differs" % (shape,)
    assert counters_zero(ws)


def test_split_full_k_transposed_a_padded_and_graph():
    """Transposed A with alpha/beta, padded and misaligned operands with a
    NaN C (nothing outside C written), and a captured graph replayed with
    eager work between the replays."""
    ws = new_ws()
    M, N, K = 5, 3000, 2500
    A, B, Cin = draw(M, N, K, seed=43, with_c=True)
    say("split full-K transposed A")
    C = run(np.ascontiguousarray(A.T), B, Cin, -1.25, 0.75, variant=VWS, workspace=ws, trans_a=True)
    ref, den = oracle.gemm(A, B, Cin, -1.25, 0.75)
    assert oracle.normalized_error(C, ref, den) <= TOL
    M, N, K = 2, 3001, 2600
    A, B, _ = draw(M, N, K, seed=44)
    say("split full-K padded")
    C = run(A, B, None, 1.0, 0.0, variant=VWS, lds=(K + 3, N + 1, N + 5), offsets=(1, 3, 2),
            check_outside=True, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C, ref, den) <= TOL
    assert counters_zero(ws)
    M, N, K = 1, 4096, 4096
    Ai, Bi, Ci = draw(M, N, K, seed=45, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bi, Ci))
    out = torch.empty_like(dC0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=VWS, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=VWS, workspace=ws)
    say("split full-K graph")
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), "replay %d" % i
        assert counters_zero(ws)


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (2, 2048, 2048), (1, 2048, 8192), (4, 4096, 4096)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_automatic_choice_with_workspace_takes_split_full_k(shape):
    """Through the workspace entry point's automatic choice these shapes take
    the split full-K form; results meet the oracle and repeat bit for bit."""
    M, N, K = shape
    need = sg.sgemm_workspace_size(0, 0, M, N, K, 1)
    v = sg.sgemm_strided_batched_ws_select_variant(0, 0, M, N, K, 1.0, 256, K, 0, 256, N, 0, 0.0, 256, N, 0, 1,
                                                   WS_BYTES)
    say("auto split full-K", shape, sg.sgemm_variant_name(v), need)
    assert v == VWS and 4096 < need <= WS_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    A, B, _ = draw(M, N, K, seed=N + K + 7)
    C1 = run(A, B, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C1, ref, den) <= TOL
    C2 = run(A, B, workspace=ws)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    assert counters_zero(ws)


# The matrix-core few-rows kernel split over K through the workspace
# (fewrows_m32_ws): 33 to 128 strips of 16 columns (two to four K chunks),
# wider strips past 2048 columns (two or four column blocks per lane), both
# orientations of B, one and two 16-row blocks, ragged N and K; past 8192
# columns the plain kernel.
VFW = sg.variant_names().index("fewrows_m32_ws")
FEW_SPLIT_CASES = [((16, 2048, 2048), False), ((16, 2048, 2048), True), ((8, 1024, 4096), False),
                   ((32, 2048, 3000), True), ((20, 1500, 2200), False), ((3, 1030, 8200), True),
                   ((8, 520, 4100), False), ((6, 3000, 4096), False), ((16, 4096, 4096), True),
                   ((24, 8000, 2048), False), ((5, 4100, 3000), False), ((9, 6000, 8192), True),
                   ((8, 9000, 2048), False)]


@pytest.mark.parametrize("case", FEW_SPLIT_CASES, ids=lambda c: "%dx%dx%d-%s" % (c[0] + ("NT" if c[1] else "NN",)))
def test_fewrows_split_against_oracle(case):
    (M, N, K), tb = case
    ws = new_ws()
    say("few-rows matrix-core split", (M, N, K), tb)
    A, B, _ = draw(M, N, K, seed=M * 3 + N + K)
    Bs = np.ascontiguousarray(B.T) if tb else B
    C1 = run(A, Bs, variant=VFW, workspace=ws, trans_b=tb)
    assert counters_zero(ws), "counters left set"
    ref, den = oracle.gemm(A, B)
    err = oracle.normalized_error(C1, ref, den)
    assert err <= TOL, "%s: normalized error %.3g" % ((M, N, K), err)
    C2 = run(A, Bs, variant=VFW, workspace=ws, trans_b=tb)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "not bitwise repeatable"
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K + 3, kind="int", with_c=True)
    Bis = np.ascontiguousarray(Bi.T) if tb else Bi
    C3 = run(Ai, Bis, Ci, 1.0, 1.0, variant=VFW, workspace=ws, trans_b=tb)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    assert oracle.exact_match(C3, ref), "%s: integer result differs" % ((M, N, K),)
    assert counters_zero(ws)


def test_fewrows_split_transposed_a_padded():
    """Transposed A with alpha/beta; padded, misaligned operands with a NaN
    C (nothing outside C written); rows past 32 in blocks of 32."""
    ws = new_ws()
    M, N, K = 12, 1600, 4100
    A, B, Cin = draw(M, N, K, seed=46, with_c=True)
    say("few-rows split transposed A")
    C = run(np.ascontiguousarray(A.T), B, Cin, 0.5, -2.0, variant=VFW, workspace=ws, trans_a=True)
    ref, den = oracle.gemm(A, B, Cin, 0.5, -2.0)
    assert oracle.normalized_error(C, ref, den) <= TOL
    M, N, K = 24, 1999, 2100
    A, B, _ = draw(M, N, K, seed=47)
    say("few-rows split padded")
    C = run(A, B, None, 1.0, 0.0, variant=VFW, lds=(K + 3, N + 1, N + 5), offsets=(1, 3, 2),
            check_outside=True, workspace=ws)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C, ref, den) <= TOL
    M, N, K = 40, 2048, 2048
    Ai, Bi, _ = draw(M, N, K, seed=48, kind="int")
    say("few-rows split row blocks")
    C = run(Ai, Bi, variant=VFW, workspace=ws)
    ref, _ = oracle.gemm(Ai, Bi)
    assert oracle.exact_match(C, ref)
    assert counters_zero(ws)


@pytest.mark.parametrize("case", [((16, 1024, 4096), False), ((24, 6144, 4096), False), ((8, 2048, 2048), True)],
                         ids=lambda c: "%dx%dx%d-%s" % (c[0] + ("NT" if c[1] else "NN",)))
def test_fewrows_split_in_a_graph(case):
    """The matrix-core few-rows split (16-column strips, and 64-column strips
    past 2048 columns) captured in a HIP graph replays exactly, with eager
    work between the replays (each replay's last chunks reset the counters)."""
    (M, N, K), tb = case
    Ai, Bi, Ci = draw(M, N, K, seed=M + N, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    Bs = np.ascontiguousarray(Bi.T) if tb else Bi
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bs, Ci))
    out = torch.empty_like(dC0)
    ws = new_ws()
    say("few-rows split in a graph", (M, N, K), tb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=VFW, workspace=ws, trans_b=tb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=VFW, workspace=ws, trans_b=tb)
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), "replay %d" % i
        assert counters_zero(ws)


@pytest.mark.parametrize("case", [((8, 1024, 8192), False), ((16, 1024, 8192), False), ((4, 1024, 4096), True),
                                  ((32, 2048, 4096), False), ((1, 1500, 16384), False),
                                  ((16, 6144, 4096), False), ((1, 3072, 8192), False)],
                         ids=lambda c: "%dx%dx%d-%s" % (c[0] + ("NT" if c[1] else "NN",)))
def test_automatic_choice_with_workspace_takes_fewrows_split(case):
    """Through the workspace entry point's automatic choice these shapes take
    the matrix-core few-rows kernel split over K, with the workspace size the
    library reports; results meet the oracle and repeat bit for bit."""
    (M, N, K), tb = case
    need = sg.sgemm_workspace_size(0, 1 if tb else 0, M, N, K, 1)
    v = sg.sgemm_strided_batched_ws_select_variant(0, 1 if tb else 0, M, N, K, 1.0, 256, K, 0, 256,
                                                   K if tb else N, 0, 0.0, 256, N, 0, 1, WS_BYTES)
    say("auto few-rows split", (M, N, K), tb, sg.sgemm_variant_name(v), need)
    assert v == VFW and 4096 < need <= WS_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    A, B, _ = draw(M, N, K, seed=N + K + 11)
    Bs = np.ascontiguousarray(B.T) if tb else B
    C1 = run(A, Bs, workspace=ws, trans_b=tb)
    ref, den = oracle.gemm(A, B)
    assert oracle.normalized_error(C1, ref, den) <= TOL
    C2 = run(A, Bs, workspace=ws, trans_b=tb)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    Ai, Bi, _ = draw(M, N, K, seed=N + K + 12, kind="int")
    Bis = np.ascontiguousarray(Bi.T) if tb else Bi
    C3 = run(Ai, Bis, workspace=ws, trans_b=tb)
    ref, _ = oracle.gemm(Ai, Bi)
    assert oracle.exact_match(C3, ref)
    assert counters_zero(ws)
