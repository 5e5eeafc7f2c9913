"""The C ABI from a plain C program (tests/c_client.c): no Python and no
torch between the caller and the library.  On the CPU the program must
compile and link against the built library without warnings; on an MI355X
its three results (sgemm, the workspace entry point, the no-alloc entry
point) must meet the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import draw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "dense_fp32_gemm_sgemm_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(out_dir):
    exe = os.path.join(str(out_dir), "c_client")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_client.c"), "-L" + LIBDIR, "-lsgemm_gfx950",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + LIBDIR,
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    return exe


def test_c_client_builds(tmp_path):
    """include/sgemm.h is plain C and the library links from C."""
    if not os.path.exists(os.path.join(LIBDIR, "libsgemm_gfx950.so")):
        pytest.skip("library not built")
    assert os.path.exists(build_client(tmp_path))


@pytest.mark.gpu
@pytest.mark.parametrize("shape,kind,alpha,beta", [((300, 260, 530), "real", 1.5, 0.5),
                                                   ((1, 4096, 4096), "int", 1.0, 1.0),
                                                   ((4095, 4097, 1023), "int", 1.0, 0.0)],
                         ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else str(x))
def test_c_client_against_oracle(tmp_path, shape, kind, alpha, beta):
    M, N, K = shape
    exe = build_client(tmp_path)
    A, B, C = draw(M, N, K, seed=M + N + K, kind=kind, with_c=True)
    src, dst = os.path.join(str(tmp_path), "in.bin"), os.path.join(str(tmp_path), "out.bin")
    with open(src, "wb") as f:
        for x in (A, B, C):
            f.write(np.ascontiguousarray(x, dtype=np.float32).tobytes())
    print("c client", shape, kind, flush=True)
    res = subprocess.run([exe, str(M), str(N), str(K), repr(alpha), repr(beta), src, dst],
                         capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    out = np.fromfile(dst, dtype=np.float32).reshape(3, M, N)
    if M * N * K <= 2 ** 31:
        ref, den = oracle.gemm(A, B, C, alpha, beta)
        for form in range(3):
            if kind == "int":
                assert oracle.exact_match(out[form], ref), "form %d" % form
            else:
                assert oracle.normalized_error(out[form], ref, den) <= 1e-5, "form %d" % form
    else:  # sampled rows and columns, every value exact (integer data)
        rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 64)), [M - 1]]))
        cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 64)), [N - 1]]))
        ref_r, _ = oracle.gemm(A, B, C, alpha, beta, rows=rows)
        ref_c, _ = oracle.gemm(A, B, C, alpha, beta, cols=cols)
        for form in range(3):
            assert oracle.exact_match(out[form][rows], ref_r), "form %d rows" % form
            assert oracle.exact_match(out[form][:, cols], ref_c), "form %d cols" % form
