"""GPU test of the entry point that allocates nothing
(sgemm_strided_batched_noalloc): called through the C ABI, it must give
bitwise the same C as the workspace entry point it stands in for
(sgemm_strided_batched_ws with a caller workspace of the same size), meet the
oracle's bars, take the split tail form where that entry point does, and keep
working on later, smaller calls, captured in a HIP graph included."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import dense_fp32_gemm_sgemm_amd as sg  # noqa: E402
from workloads import draw  # noqa: E402

pytestmark = pytest.mark.gpu

SCRATCH = 4096 + (32 << 20)   # the library's static scratch


def _call(entry, A, B, C, alpha, beta, ws=None, batch=1):
    """One call through the C ABI on the current stream; C is updated in place."""
    M, K = A.shape[-2], A.shape[-1]
    N = B.shape[-1]
    h = torch.cuda.current_stream().cuda_stream
    sa = A.stride(0) if batch > 1 else 0
    sb = B.stride(0) if batch > 1 else 0
    sc = C.stride(0) if batch > 1 else 0
    args = (0, 0, M, N, K, float(alpha), A.data_ptr(), K, sa, B.data_ptr(), N, sb, float(beta),
            C.data_ptr(), N, sc, batch)
    if entry == "ws":
        st = sg.sgemm_strided_batched_ws(*args, ws.data_ptr(), ws.numel(), h)
    else:
        st = sg.sgemm_strided_batched_noalloc(*args, h)
    assert st == sg.SGEMM_OK, sg.sgemm_status_string(st)


def _both(A, B, Cin, alpha, beta, batch=1):
    """(C from the workspace entry point, C from the no-alloc one)."""
    ws = torch.zeros(SCRATCH, dtype=torch.uint8, device="cuda")
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C1 = torch.from_numpy(Cin).cuda()
    C2 = C1.clone()
    _call("ws", dA, dB, C1, alpha, beta, ws=ws, batch=batch)
    _call("noalloc", dA, dB, C2, alpha, beta, batch=batch)
    torch.cuda.synchronize()
    return C1.cpu().numpy(), C2.cpu().numpy()


# Two calls in a row, the second smaller: both take the split tail form.
SHAPES = [(3000, 3000, 3000), (1536, 1536, 1536)]


@pytest.mark.parametrize("kind", ["real", "int"])
def test_noalloc_matches_workspace_entry_point(kind):
    for i, (M, N, K) in enumerate(SHAPES):
        v = sg.sgemm_strided_batched_ws_select_variant(0, 0, M, N, K, 1.5, 256, K, 0, 256, N, 0, 0.5, 256, N,
                                                       0, 1, SCRATCH)
        print("no-alloc", kind, (M, N, K), sg.sgemm_variant_name(v), flush=True)
        assert sg.sgemm_variant_name(v).endswith("_tail")
        A, B, Cin = draw(M, N, K, seed=900 + i, kind=kind, with_c=True)
        alpha, beta = (1.5, 0.5) if kind == "real" else (1.0, 1.0)
        C_ws, C_na = _both(A, B, Cin, alpha, beta)
        assert np.array_equal(C_ws.view(np.uint32), C_na.view(np.uint32)), "differs from the ws entry point"
        ref, den = oracle.gemm(A, B, Cin, alpha, beta)
        if kind == "int":
            assert oracle.exact_match(C_na, ref)
        else:
            assert oracle.normalized_error(C_na, ref, den) <= 1e-5


def test_noalloc_other_paths_and_memory():
    """Problems without a split (a whole number of rounds, a batch, alpha = 0)
    run through it too, and repeated calls take no device memory."""
    A, B, Cin = draw(256, 256, 256, seed=3, kind="int", with_c=True)
    C_ws, C_na = _both(A, B, Cin, 1.0, 1.0)
    assert np.array_equal(C_ws, C_na)
    Ab = np.stack([A, A[::-1].copy()])
    Bb = np.stack([B, B[:, ::-1].copy()])
    Cb = np.stack([Cin, Cin])
    C_ws, C_na = _both(Ab, Bb, Cb, 1.0, 1.0, batch=2)
    assert np.array_equal(C_ws, C_na)
    for z in range(2):
        ref, _ = oracle.gemm(Ab[z], Bb[z], Cb[z], 1.0, 1.0)
        assert oracle.exact_match(C_na[z], ref)
    dC = torch.from_numpy(Cin).cuda()
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    _call("noalloc", dA, dB, dC, 0.0, 2.0)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy(), 2.0 * Cin)
    M, N, K = SHAPES[1]
    A, B, _ = draw(M, N, K, seed=5, kind="int")
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.zeros(M, N, device="cuda")
    _call("noalloc", dA, dB, dC, 1.0, 0.0)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(5):
        _call("noalloc", dA, dB, dC, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    ref, _ = oracle.gemm(A, B)
    assert oracle.exact_match(dC.cpu().numpy(), ref)


def test_noalloc_in_a_graph():
    """Captured into a HIP graph (the caller it is meant for) and replayed
    several times with eager work in between; every replay exact."""
    M, N, K = SHAPES[0]
    Ai, Bi, Ci = draw(M, N, K, seed=21, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bi, Ci))
    out = torch.empty_like(dC0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.add(dC0, 0.0, out=out)
        _call("noalloc", dA, dB, out, 1.0, 1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)
        _call("noalloc", dA, dB, out, 1.0, 1.0)
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), "replay %d" % i
