"""CPU tests: the oracle against its pins, and the pins against planted mistakes."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import oracle_pins
from workloads import draw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.load())


# One planted mistake per build, each applied as a text patch (old -> new,
# the old text occurring exactly once) to a temporary copy of the oracle's C
# file; the committed file holds only the definition.  Each altered build
# must fail at least one pin.  The pins run in a child process so that a
# mistake which reads wild memory cannot take the test session down with it.
_ROW_LOOP = """    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) {"""
MUTANTS = {
    "beta term dropped": (
        "if (beta != 0.0) bc = beta * (double)(*cin);", "if (beta != 0.0) bc = 0.0;"),
    "B read transposed": (
        "const double p = a * (double)brow[j];",
        "const double p = (j < K && k < N) ? a * (double)B[j * ldb + k] : 0.0;"),
    "last k term dropped": (_ROW_LOOP, _ROW_LOOP.replace("k < K;", "k < K - 1;")),
    "product sign flipped": (
        "const double p = a * (double)brow[j];", "const double p = -a * (double)brow[j];"),
    "A's leading dimension ignored": (_ROW_LOOP, _ROW_LOOP.replace("A[i * lda + k]", "A[i * K + k]")),
    "|beta C| left out of the denominator": (
        "*den = (use_ab ? d : 0.0) + fabs(bc);", "*den = use_ab ? d : 0.0;"),
    "alpha applied to the beta term": (
        "*cref = ab + bc;",
        "*cref = use_ab ? alpha * (s + (beta != 0.0 ? beta * (double)(*cin) : 0.0)) : bc;"),
    "C read with B's leading dimension": (
        "const float *cin = Cin ? Cin + i * ldc + j : NULL;",
        "const float *cin = Cin ? Cin + i * ldb + j : NULL;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        text = f.read()
    assert text.count(old) == 1, "patch for %r does not apply once" % name
    src = tmp_path / "sgemm_oracle_altered.c"
    src.write_text(text.replace(old, new))
    lib = str(tmp_path / "liboracle_altered.so")
    oracle.build(output=lib, source=str(src))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert res.returncode != 0, ("planted mistake (%s) passed every pin:\n%s"
                                 % (name, res.stdout + res.stderr))


def test_committed_oracle_holds_no_planted_mistakes():
    """The committed C file is the plain definition: no build switch, and
    none of the altered texts above."""
    with open(oracle.SOURCE) as f:
        text = f.read()
    assert "#if" not in text.replace("#ifdef _OPENMP", "").replace("#ifndef", "")
    for name, (old, new) in MUTANTS.items():
        assert new not in text, name


def test_exact_match_and_normalized_error_rules():
    ref = np.array([[1.0, 0.0], [-2.0, 3.0]])
    den = np.array([[2.0, 0.0], [4.0, 3.0]])
    C = np.array([[1.0, -0.0], [-2.0, 3.0]], np.float32)
    assert oracle.exact_match(C, ref)
    assert oracle.normalized_error(C, ref, den) == 0.0
    C2 = C.copy()
    C2[0, 0] = 1.0 + 2e-5 * 2.0
    assert not oracle.exact_match(C2, ref)
    assert 1.9e-5 < oracle.normalized_error(C2, ref, den) < 2.1e-5
    C3 = C.copy()
    C3[0, 1] = 1e-30            # D == 0 demands exactly 0
    assert oracle.normalized_error(C3, ref, den) == float("inf")
    C4 = C.copy()
    C4[1, 1] = np.nan
    assert oracle.normalized_error(C4, ref, den) == float("inf")


def test_fp32_accumulation_is_within_tolerance_but_not_exact():
    """A sequential fp32 dot product on uniform[-1,1] data passes the 1e-5 bar
    with wide margin, and an fp16-rounded-input product fails it: the metric
    separates strict FP32 from reduced-precision inputs."""
    A, B, _ = draw(64, 48, 1024, seed=1)
    ref, den = oracle.gemm(A, B)
    acc = np.zeros((64, 48), np.float32)
    for k in range(A.shape[1]):
        acc = (acc + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    err = oracle.normalized_error(acc, ref, den)
    assert err < 1e-6
    Ah = A.astype(np.float16).astype(np.float32)
    Bh = B.astype(np.float16).astype(np.float32)
    low = (Ah.astype(np.float64) @ Bh.astype(np.float64)).astype(np.float32)
    assert oracle.normalized_error(low, ref, den) > 1e-5


def test_integer_inputs_are_exact_in_fp32():
    """On {-4..4} inputs an fp32 accumulation reproduces C_ref exactly."""
    A, B, C = draw(32, 40, 4096, seed=2, kind="int", with_c=True)
    ref, _ = oracle.gemm(A, B, C, 1.0, 1.0)
    acc = np.zeros((32, 40), np.float32)
    for k in range(A.shape[1]):
        acc = (acc + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    out = (acc + C).astype(np.float32)
    assert oracle.exact_match(out, ref)


def test_threads_reported():
    assert oracle.max_threads() >= 1
