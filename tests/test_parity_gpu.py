"""GPU parity: the HIP SGEMM against the fp64 CPU oracle, through the C ABI.

Bars (from the operation's definition and the tolerance it is held to):
  * integer inputs in {-4..4}: every partial sum is an integer below 2^24, so
    the fp32 result must equal the oracle exactly;
  * real inputs: max |C - C_ref| / (sum_k |A_ik||B_kj| + |beta C_ij|) <= 1e-5;
  * permutation inputs: the product only moves values, so it is exact and
    pins the matrix-core lane maps.
Every kernel variant is checked on small shapes that span several tiles and a
ragged tail; the full-size workloads run through the automatic choice, which
is the launch configuration the benchmark times.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import dense_fp32_gemm_sgemm_amd as sg  # noqa: E402
from tests.gpu_util import run  # noqa: E402
from workloads import (ACCUM, ACCUM_INT, HEADLINE, SMALL, SMALL_INT, draw,  # noqa: E402
                       draw_workload, ragged_workloads, shard_workloads, sweep_workloads)

pytestmark = pytest.mark.gpu

TOL = 1e-5
VARIANTS = list(range(sg.sgemm_num_variants()))
VNAMES = [sg.sgemm_variant_name(v) for v in VARIANTS]


def say(*a):
    print(*a, flush=True)


def check_real(C, A, B, Cin, alpha, beta, what):
    ref, den = oracle.gemm(A, B, Cin, alpha, beta)
    err = oracle.normalized_error(C, ref, den)
    assert err <= TOL, "%s: normalized error %.3g > %g" % (what, err, TOL)
    return err


def check_exact(C, A, B, Cin, alpha, beta, what):
    ref, _ = oracle.gemm(A, B, Cin, alpha, beta)
    bad = np.argwhere(C.astype(np.float64) != ref)
    assert bad.size == 0, "%s: %d mismatches, first at %s (%r vs %r)" % (
        what, len(bad), tuple(bad[0]), C[tuple(bad[0])], ref[tuple(bad[0])])


# ---------------------------------------------------------------- every variant

@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_permutation_pins_lane_maps(variant):
    """A = P (a row permutation) gives P@B exactly; B = Q permutes columns."""
    rng = np.random.default_rng(31)
    M = K = 200
    N = 328
    perm = rng.permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1.0
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    say("perm rows", VNAMES[variant])
    C = run(P, B, variant=variant)
    assert np.array_equal(C, B[perm]), VNAMES[variant]
    q = rng.permutation(N)
    Q = np.zeros((N, N), np.float32)
    Q[q, np.arange(N)] = 1.0
    A = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    say("perm cols", VNAMES[variant])
    C = run(A, Q, variant=variant)
    assert np.array_equal(C, A[:, q]), VNAMES[variant]


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_small_config_every_variant(variant):
    """256^3, alpha=1, beta=0: real inputs to 1e-5, integer copy exact."""
    A, B, _ = draw_workload(SMALL)
    say("small real", VNAMES[variant])
    C = run(A, B, variant=variant)
    check_real(C, A, B, None, 1.0, 0.0, VNAMES[variant])
    Ai, Bi, _ = draw_workload(SMALL_INT)
    say("small int", VNAMES[variant])
    C = run(Ai, Bi, variant=variant)
    check_exact(C, Ai, Bi, None, 1.0, 0.0, VNAMES[variant])


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
@pytest.mark.parametrize("shape", [(300, 200, 100), (129, 257, 33), (64, 64, 64), (65, 63, 17),
                                   (520, 130, 1000)])
def test_ragged_every_variant(variant, shape):
    """Shapes that cut tiles in M, N and K; accumulate form (alpha, beta)."""
    M, N, K = shape
    A, B, Cin = draw(M, N, K, seed=M + N + K, with_c=True)
    say("ragged", shape, VNAMES[variant])
    C = run(A, B, Cin, 1.5, 0.5, variant=variant, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "%s %s" % (VNAMES[variant], shape))
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=variant)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s int" % (VNAMES[variant], shape))


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_bruteforce_tiny_shapes(variant):
    """Every (M,N,K) in [1..9]^3 and {63,64,65}^3, integer data, exact."""
    shapes = [(m, n, k) for m in range(1, 10) for n in range(1, 10) for k in range(1, 10)]
    shapes += [(m, n, k) for m in (63, 64, 65) for n in (63, 64, 65) for k in (63, 64, 65)]
    say("bruteforce", VNAMES[variant], len(shapes), "shapes")
    for (M, N, K) in shapes:
        A, B, Cin = draw(M, N, K, seed=1000 + M * 100 + N * 10 + K, kind="int", with_c=True)
        C = run(A, B, Cin, 1.0, 1.0, variant=variant)
        check_exact(C, A, B, Cin, 1.0, 1.0, "%s (%d,%d,%d)" % (VNAMES[variant], M, N, K))


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_leading_dims_alignment_and_canaries(variant):
    """Padded leading dimensions with NaN gaps, misaligned bases; nothing
    outside C's elements is written and no gap is read."""
    M, N, K = 150, 140, 70
    A, B, Cin = draw(M, N, K, seed=77, kind="int", with_c=True)
    cases = [((K + 5, N + 3, N + 7), (0, 0, 0)),
             ((K + 4, N + 4, N + 4), (0, 0, 0)),
             ((K, N, N), (1, 2, 3)),
             ((K + 3, N + 1, N + 2), (3, 1, 2))]
    for lds, offs in cases:
        say("ld/offset", VNAMES[variant], lds, offs)
        C = run(A, B, Cin, 1.0, 1.0, variant=variant, lds=lds, offsets=offs, check_outside=True)
        check_exact(C, A, B, Cin, 1.0, 1.0, "%s lds=%s offs=%s" % (VNAMES[variant], lds, offs))


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_offsets_beyond_32_bits(variant):
    """A leading dimension of 2^27 with 17 rows puts the last row 2^31
    elements (8 GiB) past the first: any 32-bit element index on the path of
    A, B or C would wrap.  Integer data, exact."""
    big = 1 << 27
    for which, (M, N, K) in (("A", (17, 192, 64)), ("B", (96, 128, 17)), ("C", (17, 160, 48))):
        A, B, Cin = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
        lds = (big if which == "A" else None, big if which == "B" else None,
               big if which == "C" else None)
        say("64-bit offsets", VNAMES[variant], which)
        C = run(A, B, Cin, 1.0, 1.0, variant=variant, lds=lds)
        check_exact(C, A, B, Cin, 1.0, 1.0, "%s ld(%s)=2^27" % (VNAMES[variant], which))
        torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
@pytest.mark.parametrize("ops", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
def test_transposed_operands_every_variant(variant, ops):
    """op(A), op(B) in {N, T}: the stored matrices are the transposes; the
    oracle gets op(A) and op(B) written out, the GPU the stored matrices."""
    ta, tb = ops
    for (M, N, K), pad in (((300, 200, 100), False), ((129, 257, 33), False), ((65, 63, 17), True),
                           ((520, 130, 1000), False)):
        A, B, Cin = draw(M, N, K, seed=M + N + K + 7, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        # padded case: leading dimensions longer than the stored rows
        lds = (As.shape[1] + 6, Bs.shape[1] + 3, N + 7) if pad else (None, None, None)
        say("transposed", ops, (M, N, K), VNAMES[variant])
        C = run(As, Bs, Cin, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, lds=lds,
                check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "%s %s %s" % (VNAMES[variant], ops, (M, N, K)))
        Ai, Bi, Ci = draw(M, N, K, seed=M + N + K + 7, kind="int", with_c=True)
        C = run(np.ascontiguousarray(Ai.T) if ta else Ai, np.ascontiguousarray(Bi.T) if tb else Bi,
                Ci, 1.0, 1.0, variant=variant, trans_a=ta, trans_b=tb)
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s %s int" % (VNAMES[variant], ops, (M, N, K)))


@pytest.mark.parametrize("ops", [(False, False), (False, True), (True, False), (True, True)],
                         ids=["NN", "NT", "TN", "TT"])
def test_transposed_operands_full_size(ops):
    """4096^3 and 1x4096x4096 through the automatic choice for every transpose
    combination; 4096^3 checked on 128 sampled whole rows and columns."""
    ta, tb = ops
    A, B, _ = draw(4096, 4096, 4096, seed=21)
    say("transposed 4096^3", ops)
    C = run(np.ascontiguousarray(A.T) if ta else A, np.ascontiguousarray(B.T) if tb else B,
            trans_a=ta, trans_b=tb)
    _sampled_check(A, B, C, 1.0, 0.0, None, 128, 128, 21, "4096^3 %s" % (ops,))
    A, B, _ = draw(1, 4096, 4096, seed=22)
    C = run(np.ascontiguousarray(A.T) if ta else A, np.ascontiguousarray(B.T) if tb else B,
            trans_a=ta, trans_b=tb)
    check_real(C, A, B, None, 1.0, 0.0, "1x4096x4096 %s" % (ops,))


def test_column_major_via_transposition_identity():
    """A column-major C = A*B is the row-major call with the operands swapped."""
    M, N, K = 300, 200, 150
    A, B, _ = draw(M, N, K, seed=23)
    # column-major storage of A (M x K) is the row-major storage of A^T (K x M)
    A_cm = np.ascontiguousarray(A.T)
    B_cm = np.ascontiguousarray(B.T)
    say("column-major")
    Ct = run(B_cm, A_cm)            # (B^T) (A^T) = (AB)^T, N x M row-major = C column-major
    check_real(np.ascontiguousarray(Ct.T), A, B, None, 1.0, 0.0, "column-major")


def run_batched(A, B, C, alpha, beta, *, variant=-1, trans_a=False, trans_b=False, shared_b=False,
                gap=0):
    """Strided-batched call on stacked slices (numpy (batch, rows, cols));
    `gap` extra NaN floats between consecutive slices, `shared_b` passes one
    B with stride 0.  Returns C as numpy and checks the gaps stay NaN."""
    batch = C.shape[0]

    def dev(X, gap_):
        b, r, c = X.shape
        stride = r * c + gap_
        buf = torch.full((b * stride + 16,), float("nan"), dtype=torch.float32, device="cuda")
        view = torch.as_strided(buf, (b, r, c), (stride, c, 1), 8)
        view.copy_(torch.from_numpy(np.ascontiguousarray(X)).cuda())
        return buf, view

    _, dA = dev(A, gap)
    if shared_b:
        _, dB1 = dev(B[:1], 0)
        dB = dB1.expand(batch, -1, -1)
    else:
        _, dB = dev(B, gap)
    bufC, dC = dev(C, gap)
    sg.gemm_batched(dA, dB, dC, alpha, beta, variant=variant, trans_a=trans_a, trans_b=trans_b)
    torch.cuda.synchronize()
    mask = torch.ones_like(bufC, dtype=torch.bool)
    idx = torch.as_strided(torch.arange(bufC.numel(), device="cuda"), dC.shape, dC.stride(), 8)
    mask[idx.reshape(-1)] = False
    assert bool(torch.isnan(bufC[mask]).all().item()), "memory outside the C slices was written"
    return dC.cpu().numpy()


def check_batched(C, A, B, Cin, alpha, beta, what, exact=False, ta=False, tb=False):
    for z in range(C.shape[0]):
        a = np.ascontiguousarray(A[z].T) if ta else A[z]
        b = np.ascontiguousarray(B[z].T) if tb else B[z]
        if exact:
            check_exact(C[z], a, b, Cin[z], alpha, beta, "%s slice %d" % (what, z))
        else:
            check_real(C[z], a, b, Cin[z], alpha, beta, "%s slice %d" % (what, z))


SCHED = [v for v in VARIANTS if VNAMES[v].endswith("_sched")]


@pytest.mark.parametrize("variant", SCHED, ids=[VNAMES[v] for v in SCHED])
@pytest.mark.parametrize("shape", [(300, 264, 64), (256, 256, 32), (520, 392, 96), (600, 500, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_sched_path_shapes_and_orientations(variant, shape):
    """Shapes that meet the ordered-loop kernel's preconditions (the tile
    inside C, K at least one slab) for at least the smaller tiles: tiles
    shifted back inside C on both edges, a single slab, every operand
    orientation, the accumulate form; real to 1e-5 and integer data exactly."""
    M, N, K = shape
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        A, B, Cin = draw(M, N, K, seed=M + 7 * N + K, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        say("sched", VNAMES[variant], shape, ta, tb)
        C = run(As, Bs, Cin, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "%s %s %s%s" % (VNAMES[variant], shape, ta, tb))
        Ai, Bi, Ci = draw(M, N, K, seed=M + 7 * N + K, kind="int", with_c=True)
        Ais = np.ascontiguousarray(Ai.T) if ta else Ai
        Bis = np.ascontiguousarray(Bi.T) if tb else Bi
        C = run(Ais, Bis, Ci, 1.0, 1.0, variant=variant, trans_a=ta, trans_b=tb)
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s %s%s int" % (VNAMES[variant], shape, ta, tb))


@pytest.mark.parametrize("variant", SCHED, ids=[VNAMES[v] for v in SCHED])
@pytest.mark.parametrize("shape", [(300, 270, 70), (260, 301, 33), (520, 390, 161)],
                         ids=lambda s: "x".join(map(str, s)))
def test_sched_path_ragged_k_and_unaligned(variant, shape):
    """K that is not a multiple of the slab depth (later slabs start early so
    the last ends at K; the k two slabs share are zero in the first), operands and C at
    4-byte but not 16-byte aligned addresses with odd leading dimensions, and N
    not a multiple of 4 (column groups of the permuted B straddling a shifted
    tile's edge); every orientation, the accumulate form; nothing outside C is
    written."""
    M, N, K = shape
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        A, B, Cin = draw(M, N, K, seed=M + 3 * N + K, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        lds = (As.shape[1] + 3, Bs.shape[1] + 1, N + 5)
        say("sched ragged", VNAMES[variant], shape, ta, tb)
        C = run(As, Bs, Cin, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, lds=lds,
                offsets=(1, 3, 2), check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "%s %s %s%s" % (VNAMES[variant], shape, ta, tb))
        Ai, Bi, Ci = draw(M, N, K, seed=M + 3 * N + K, kind="int", with_c=True)
        Ais = np.ascontiguousarray(Ai.T) if ta else Ai
        Bis = np.ascontiguousarray(Bi.T) if tb else Bi
        C = run(Ais, Bis, Ci, 1.0, 1.0, variant=variant, trans_a=ta, trans_b=tb, lds=lds,
                offsets=(2, 1, 3))
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s %s%s int" % (VNAMES[variant], shape, ta, tb))


@pytest.mark.parametrize("variant", SCHED, ids=[VNAMES[v] for v in SCHED])
def test_sched_misaligned_c_rows(variant):
    """Rows of C that do not start on a 16-byte boundary keep the vector
    stores of the ordered loop's epilogue: an odd N (the last tile shifted
    back by an odd number of columns), an odd leading dimension of C and a C
    that starts one float into its buffer, every operand orientation, beta
    != 0 (the old C read as a vector too); real to 1e-5, integer data
    exactly, nothing outside C written."""
    for (M, N, K) in ((300, 263, 64), (257, 301, 96)):
        for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
            A, B, Cin = draw(M, N, K, seed=M + 3 * N + K, with_c=True)
            As = np.ascontiguousarray(A.T) if ta else A
            Bs = np.ascontiguousarray(B.T) if tb else B
            say("sched misaligned C", VNAMES[variant], (M, N, K), ta, tb)
            C = run(As, Bs, Cin, -1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, check_outside=True)
            check_real(C, A, B, Cin, -1.5, 0.5, "%s %s %s%s" % (VNAMES[variant], (M, N, K), ta, tb))
            C = run(As, Bs, Cin, -1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb,
                    lds=(None, None, N + 1), offsets=(0, 0, 1), check_outside=True)
            check_real(C, A, B, Cin, -1.5, 0.5, "%s %s %s%s ldc+1" % (VNAMES[variant], (M, N, K), ta, tb))
            Ai, Bi, Ci = draw(M, N, K, seed=M + 3 * N + K, kind="int", with_c=True)
            Ais = np.ascontiguousarray(Ai.T) if ta else Ai
            Bis = np.ascontiguousarray(Bi.T) if tb else Bi
            C = run(Ais, Bis, Ci, 1.0, 1.0, variant=variant, trans_a=ta, trans_b=tb,
                    lds=(None, None, N + 1), offsets=(0, 0, 1))
            check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s %s%s int" % (VNAMES[variant], (M, N, K), ta, tb))


@pytest.mark.parametrize("shape", [(64, 64, 4096), (100, 130, 3001), (70, 200, 1290), (128, 192, 2048)],
                         ids=lambda s: "x".join(map(str, s)))
def test_sched_split_k(shape):
    """The ordered loop with K split over workgroups (few tiles, long K): 16
    ranges of one tile, a ragged last range (3001), a short rest folded into
    the range before (1290 = 4 x 320 + 10), every orientation, beta != 0 (C
    scaled first), a padded / misaligned copy; real to 1e-5, integer data
    exactly (atomic adds of integers are exact in any order)."""
    M, N, K = shape
    v = VNAMES.index("mfma16_64x64x64_4x2_sched_splitk")
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        A, B, Cin = draw(M, N, K, seed=M + N + K, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        say("sched split", shape, ta, tb)
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb, check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "split %s %s%s" % (shape, ta, tb))
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb,
                lds=(As.shape[1] + 1, Bs.shape[1] + 3, N + 2), offsets=(3, 1, 2), check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "split %s %s%s padded" % (shape, ta, tb))
        Ai, Bi, Ci = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
        Ais = np.ascontiguousarray(Ai.T) if ta else Ai
        Bis = np.ascontiguousarray(Bi.T) if tb else Bi
        C = run(Ais, Bis, Ci, 1.0, 1.0, variant=v, trans_a=ta, trans_b=tb)
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "split %s %s%s int" % (shape, ta, tb))


@pytest.mark.parametrize("name", ["mfma16_64x64x64_4x2_sched_splitk", "mfma16_64x64x64_4x2_pipe_splitk"])
def test_split_k_batched_and_nan_c(name):
    """K split over workgroups together with a strided batch (blockIdx.y the
    range, blockIdx.z the slice; slices with gaps), integer data exactly; and
    beta = 0 over a NaN-filled C, which the scaling launch must overwrite with
    zeros before the ranges add into it."""
    v = VNAMES.index(name)
    rng = np.random.default_rng(77)
    batch, M, N, K = 3, 64, 96, 2048
    Ai = rng.integers(-4, 5, (batch, M, K)).astype(np.float32)
    Bi = rng.integers(-4, 5, (batch, K, N)).astype(np.float32)
    Ci = rng.integers(-4, 5, (batch, M, N)).astype(np.float32)
    say("split batched", name)
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=v, gap=5)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, name + " batched", exact=True)
    A, B, _ = draw(M, N, K, seed=78)
    say("split nan C", name)
    C = run(A, B, None, 1.0, 0.0, variant=v, check_outside=True)  # C starts NaN
    check_real(C, A, B, None, 1.0, 0.0, name + " beta 0 over NaN")


@pytest.mark.parametrize("variant", SCHED, ids=[VNAMES[v] for v in SCHED])
def test_sched_path_inf_in_repeated_k(variant):
    """Infs at a k that two slabs cover when the slab depth does not divide K,
    one in A (row 7) and one in B (column 5): one of the two copies must be
    zero in both operands, so C is +-Inf exactly in row 7 and column 5, as
    the definition gives, never NaN (a zero in one operand only would make
    0 * Inf there)."""
    M, N, K = 300, 264, 70
    rng = np.random.default_rng(5)
    A = (rng.integers(1, 5, (M, K)) * rng.choice([-1, 1], (M, K))).astype(np.float32)
    B = rng.integers(1, 5, (K, N)).astype(np.float32)   # positive: no Inf - Inf
    k = 20          # among the k that slab 0 zeroes for 32- and 64-deep slabs ([6, 32), [6, 64))
    A[7, k] = np.inf
    B[k, 5] = np.inf
    say("sched inf", VNAMES[variant])
    C = run(A, B, variant=variant)
    ref, _ = oracle.gemm(A, B, None, 1.0, 0.0)
    assert not np.isnan(ref).any()
    assert np.array_equal(C.astype(np.float64), ref), VNAMES[variant]


@pytest.mark.parametrize("variant", SCHED, ids=[VNAMES[v] for v in SCHED])
def test_sched_path_permutation_and_batch(variant):
    """Lane maps of the ordered loop pinned exactly (A = P with K = 256, N a
    multiple of 4 past the tile), and a strided batch with 16-byte strides."""
    rng = np.random.default_rng(41)
    M = K = 256
    N = 264
    perm = rng.permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1.0
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    say("sched perm", VNAMES[variant])
    C = run(P, B, variant=variant)
    assert np.array_equal(C, B[perm]), VNAMES[variant]
    Ai = rng.integers(-4, 5, (3, 260, 128)).astype(np.float32)
    Bi = rng.integers(-4, 5, (3, 128, 256)).astype(np.float32)
    Ci = rng.integers(-4, 5, (3, 260, 256)).astype(np.float32)
    say("sched batch", VNAMES[variant])
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=variant, gap=4)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, VNAMES[variant] + " batch", exact=True)
    # slice strides that are not whole 16-byte vectors: aligned first slice and
    # leading dimensions, later slices only 4-byte aligned
    say("sched batch odd stride", VNAMES[variant])
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=variant, gap=1)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, VNAMES[variant] + " batch odd stride", exact=True)


@pytest.mark.parametrize("variant", VARIANTS, ids=VNAMES)
def test_strided_batched_every_variant(variant):
    """Three slices with gaps between them, every transpose combination, a
    shared B (stride 0); real data to the tolerance, integer data exactly."""
    rng = np.random.default_rng(41)
    for ta, tb in ((False, False), (True, False), (False, True), (True, True)):
        M, N, K, batch = 131, 70, 97, 3
        A = rng.uniform(-1, 1, (batch, K, M) if ta else (batch, M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (batch, N, K) if tb else (batch, K, N)).astype(np.float32)
        C = rng.standard_normal((batch, M, N)).astype(np.float32)
        say("batched", VNAMES[variant], ta, tb)
        out = run_batched(A, B, C, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, gap=5)
        check_batched(out, A, B, C, 1.5, 0.5, VNAMES[variant], ta=ta, tb=tb)
    Ai = rng.integers(-4, 5, (4, 65, 40)).astype(np.float32)
    Bi = rng.integers(-4, 5, (4, 40, 33)).astype(np.float32)
    Bi[:] = Bi[0]
    Ci = rng.integers(-4, 5, (4, 65, 33)).astype(np.float32)
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=variant, shared_b=True)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, VNAMES[variant] + " shared B", exact=True)


@pytest.mark.parametrize("shape", [(64, 512, 512, 512), (256, 64, 64, 64), (8, 1024, 1024, 1024),
                                   (2, 1, 4096, 4096), (1024, 128, 128, 128), (256, 256, 256, 256),
                                   (4096, 32, 32, 32), (128, 200, 300, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_strided_batched_automatic(shape):
    batch, M, N, K = shape
    rng = np.random.default_rng(batch + M)
    A = rng.uniform(-1, 1, (batch, M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (batch, K, N)).astype(np.float32)
    C = np.full((batch, M, N), np.nan, np.float32)
    say("batched auto", shape)
    out = run_batched(A, B, C, 1.0, 0.0)
    check_batched(out, A, B, np.zeros_like(C), 1.0, 0.0, "auto %s" % (shape,))


def _random_problem(rng):
    """A seeded random problem: dimensions near powers of two and tile edges
    or anywhere up to ~700 (or, for a third of the problems, 1500..4200 with
    K below 600, so that the large tiles run), random operand orientations, a
    batch of one to three, random alpha and beta, packed or padded leading
    dimensions."""
    def dim():
        if rng.random() < 0.5:
            return int(max(1, rng.choice([16, 32, 64, 128, 256, 512]) + rng.integers(-2, 3)))
        return int(rng.integers(1, 700))

    def big():
        if rng.random() < 0.5:
            return int(256 * rng.integers(6, 17) + rng.choice([0, 0, 4, -4, 3]))
        return int(rng.integers(1500, 4200))
    if rng.random() < 0.35:  # enough tiles for the 128x128 and 256x256 families
        M, N, K = big(), big(), int(rng.integers(1, 600))
    else:
        M, N, K = dim(), dim(), dim()
    ta, tb = bool(rng.random() < 0.3), bool(rng.random() < 0.3)
    batch = int(rng.choice([1, 1, 2, 3]))
    alpha = float(rng.choice([1.0, 1.5, -0.5]))
    beta = float(rng.choice([0.0, 1.0, 0.5]))
    pad = int(rng.choice([0, 0, 1, 4]))
    return M, N, K, ta, tb, batch, alpha, beta, pad


@pytest.mark.parametrize("seed", range(80))
def test_random_problems_automatic(seed):
    """Random shapes, orientations, batches and scalars through the automatic
    choice (every kernel family and its fallbacks get some), real data to
    1e-5 against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    M, N, K, ta, tb, batch, alpha, beta, pad = _random_problem(rng)
    say("random", seed, M, N, K, ta, tb, batch, alpha, beta, pad)
    if batch == 1:
        A, B, Cin = draw(M, N, K, seed=seed, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        lds = (As.shape[1] + pad, Bs.shape[1] + pad, N + pad)
        C = run(As, Bs, Cin, alpha, beta, trans_a=ta, trans_b=tb, lds=lds, check_outside=True)
        check_real(C, A, B, Cin, alpha, beta, "random %d" % seed)
    else:
        A = rng.uniform(-1, 1, (batch, K, M) if ta else (batch, M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (batch, N, K) if tb else (batch, K, N)).astype(np.float32)
        Cin = rng.standard_normal((batch, M, N)).astype(np.float32)
        out = run_batched(A, B, Cin, alpha, beta, trans_a=ta, trans_b=tb, gap=pad)
        check_batched(out, A, B, Cin, alpha, beta, "random %d" % seed, ta=ta, tb=tb)


def test_strided_batched_more_slices_than_one_grid():
    """65,543 slices: more than one grid's worth (65,535), so the entry point
    splits the batch into launches."""
    rng = np.random.default_rng(43)
    batch, M, N, K = 65543, 2, 3, 4
    A = rng.integers(-4, 5, (batch, M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (batch, K, N)).astype(np.float32)
    C = rng.integers(-4, 5, (batch, M, N)).astype(np.float32)
    say("batched 65543 slices")
    out = run_batched(A, B, C, 1.0, 1.0)
    check_batched(out, A, B, C, 1.0, 1.0, "65543 slices", exact=True)


# ---------------------------------------------------------------- special cases

def test_beta_zero_ignores_nan_in_c():
    A, B, _ = draw(200, 180, 90, seed=5)
    say("beta=0 with NaN C")
    C = run(A, B, None, 1.0, 0.0)
    assert np.all(np.isfinite(C))
    check_real(C, A, B, None, 1.0, 0.0, "beta=0")


def test_alpha_zero_and_k_zero_scale_c():
    rng = np.random.default_rng(6)
    Cin = rng.integers(-4, 5, (70, 90)).astype(np.float32)
    A = np.full((70, 30), np.nan, np.float32)   # must not be read
    B = np.full((30, 90), np.nan, np.float32)
    say("alpha=0")
    C = run(A, B, Cin, 0.0, 0.5)
    assert np.array_equal(C, 0.5 * Cin)
    C = run(A, B, Cin, 0.0, 0.0)
    assert np.all(C == 0)
    C = run(A, B, Cin, 0.0, 1.0)
    assert np.array_equal(C, Cin)
    say("K=0")
    C = run(np.zeros((70, 0), np.float32), np.zeros((0, 90), np.float32), Cin, 2.0, -1.5)
    assert np.array_equal(C, -1.5 * Cin)


def test_empty_problems_are_noops():
    for (M, N, K) in ((0, 5, 5), (5, 0, 5), (0, 0, 0)):
        A, B, _ = draw(M, N, K, seed=1)
        C = run(A, B, np.ones((M, N), np.float32), 1.0, 1.0)
        assert C.shape == (M, N)


def test_nan_in_a_poisons_its_row_only():
    A, B, _ = draw(130, 140, 60, seed=8)
    A[7, 13] = np.nan
    say("NaN in A")
    C = run(A, B, np.zeros((130, 140), np.float32), 1.0, 0.0)
    assert np.all(np.isnan(C[7]))
    rest = np.delete(C, 7, axis=0)
    assert np.all(np.isfinite(rest))


# Variants whose K-sum order is fixed; the split-K and few-rows variants add
# partial sums with atomics in an order the hardware chooses.
DETERMINISTIC = [v for v in VARIANTS if not (VNAMES[v].endswith("_splitk") or VNAMES[v].startswith("skinny"))]
UNORDERED = [v for v in VARIANTS if v not in DETERMINISTIC]


@pytest.mark.parametrize("variant", DETERMINISTIC, ids=[VNAMES[v] for v in DETERMINISTIC])
def test_repeatable_bitwise(variant):
    A, B, Cin = draw(700, 600, 900, seed=12, with_c=True)
    say("repeatability", VNAMES[variant])
    C1 = run(A, B, Cin, 1.5, 0.5, variant=variant)
    C2 = run(A, B, Cin, 1.5, 0.5, variant=variant)
    assert np.array_equal(C1, C2)


def test_automatic_choice_repeatable_at_headline_size():
    A, B, _ = draw(4096, 4096, 4096, seed=3)
    say("repeatability 4096^3")
    assert np.array_equal(run(A, B), run(A, B))


@pytest.mark.parametrize("variant", UNORDERED, ids=[VNAMES[v] for v in UNORDERED])
@pytest.mark.parametrize("shape", [(700, 600, 3000), (256, 256, 4096), (8, 1000, 2500), (1, 4097, 4096),
                                   (3, 130, 777)])
def test_split_reductions(variant, shape):
    """Split-K and few-rows kernels: K split across workgroups, partial sums
    added with atomics after C is scaled by beta."""
    M, N, K = shape
    A, B, Cin = draw(M, N, K, seed=M + N + K, with_c=True)
    say("split", VNAMES[variant], shape)
    C = run(A, B, Cin, 1.5, 0.5, variant=variant, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "%s %s" % (VNAMES[variant], shape))
    C = run(A, B, None, 1.0, 0.0, variant=variant)   # beta = 0 over NaN-filled C
    check_real(C, A, B, None, 1.0, 0.0, "%s %s beta=0" % (VNAMES[variant], shape))
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=variant)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s int" % (VNAMES[variant], shape))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_few_rows_automatic(M):
    """Matrix-vector-like shapes through the automatic choice, including a
    misaligned B (ld not a multiple of 4)."""
    A, B, Cin = draw(M, 3001, 2049, seed=M, with_c=True)
    say("few rows", M)
    C = run(A, B, Cin, 2.0, -1.0, check_outside=True)
    check_real(C, A, B, Cin, 2.0, -1.0, "M=%d" % M)
    C = run(A, B, Cin, 2.0, -1.0, lds=(2049 + 3, 3001 + 2, 3001 + 1), offsets=(1, 2, 3), check_outside=True)
    check_real(C, A, B, Cin, 2.0, -1.0, "M=%d padded" % M)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("NK", [(2053, 1), (2048, 33), (4096, 4097), (3000, 250)],
                         ids=lambda t: "N%dK%d" % t)
def test_few_rows_full_k_strips(M, NK):
    """The few-rows kernel's full-K strip form (at least 64 strips of 32
    columns, moderate B): K tails that leave the last sweep partial (K = 1
    included), a ragged and misaligned column edge, a transposed A, the
    accumulate form; real data to 1e-5, integer data exactly."""
    N, K = NK
    v = VNAMES.index("skinny_m8")
    A, B, Cin = draw(M, N, K, seed=M * 31 + N + K, with_c=True)
    say("full-K strips", M, N, K)
    C = run(A, B, Cin, 1.5, 0.5, variant=v, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "M=%d N=%d K=%d" % (M, N, K))
    C = run(A, B, Cin, 1.5, 0.5, variant=v, lds=(K + 3, N + 1, N + 2), offsets=(1, 3, 2),
            check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "M=%d N=%d K=%d padded" % (M, N, K))
    C = run(np.ascontiguousarray(A.T), B, Cin, 1.5, 0.5, variant=v, trans_a=True, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "M=%d N=%d K=%d TA" % (M, N, K))
    Ai, Bi, Ci = draw(M, N, K, seed=M * 31 + N + K, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=v)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "M=%d N=%d K=%d int" % (M, N, K))


@pytest.mark.parametrize("shape", [(3, 1024, 4100), (8, 1000, 3001), (1, 2048, 4097)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_rows_vector_loads_on_misaligned_rows(shape):
    """The few-rows kernels forced with N a multiple of 4 but rows of A and B
    that do not start on 16-byte boundaries (odd leading dimensions, bases
    one or three floats in): four consecutive floats still go as one vector.
    K split over workgroups (fewer than 64 strips of 32 columns) and the
    full-K strips, beta != 0; real to 1e-5, integer data exactly."""
    M, N, K = shape
    v = VNAMES.index("skinny_m8")
    A, B, Cin = draw(M, N, K, seed=M + N + K, with_c=True)
    say("few rows misaligned", shape)
    C = run(A, B, Cin, -0.75, 0.5, variant=v, lds=(K + 1, N + 1, N + 3), offsets=(3, 1, 2),
            check_outside=True)
    check_real(C, A, B, Cin, -0.75, 0.5, "%s padded" % (shape,))
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=v, lds=(K + 1, N + 1, N + 3), offsets=(3, 1, 2))
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s int padded" % (shape,))


@pytest.mark.parametrize("N", [1, 5, 16])
@pytest.mark.parametrize("MK", [(16, 1), (100, 15), (1000, 33), (333, 4099), (64, 20000)],
                         ids=lambda t: "M%dK%d" % t)
def test_few_columns_kernel(N, MK):
    """The few-columns kernel forced: K ranges that leave the last wave empty
    or partial (K = 1 included), ragged rows, every operand orientation, a
    padded / misaligned copy, the accumulate form; real data to 1e-5 and
    integer data exactly."""
    M, K = MK
    v = VNAMES.index("narrow_n16")
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        A, B, Cin = draw(M, N, K, seed=M + 3 * N + K, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        say("few columns", M, N, K, ta, tb)
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb, check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "M=%d N=%d K=%d %s%s" % (M, N, K, ta, tb))
    A, B, Cin = draw(M, N, K, seed=M + 3 * N + K, with_c=True)
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb,
                lds=(As.shape[1] + 1, Bs.shape[1] + 3, N + 2), offsets=(3, 1, 2), check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "M=%d N=%d K=%d %s%s padded" % (M, N, K, ta, tb))
    Ai, Bi, Ci = draw(M, N, K, seed=M + 3 * N + K, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=v)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "M=%d N=%d K=%d int" % (M, N, K))
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=v, lds=(K + 1, N + 3, N + 2), offsets=(3, 1, 2))
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "M=%d N=%d K=%d int padded" % (M, N, K))


@pytest.mark.parametrize("shape", [(9, 100, 33), (16, 1000, 1000), (1, 4099, 5), (12, 4096, 1),
                                   (16, 257, 4099), (24, 4099, 33), (32, 257, 1000), (37, 300, 70),
                                   (12, 16384, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_rows_matrix_core_kernel(shape):
    """The matrix-core few-rows kernel forced: K ranges that leave the last
    wave empty or partial (K = 1 included), N not a multiple of the columns a
    lane loads, every operand orientation, a padded / misaligned copy, one
    and two 16-row blocks, row blocks past 32 (M = 37), the accumulate form;
    real data to 1e-5 and integer data exactly."""
    M, N, K = shape
    v = VNAMES.index("fewrows_m32")
    for ta, tb in ((False, False), (False, True), (True, False), (True, True)):
        A, B, Cin = draw(M, N, K, seed=M + 5 * N + K, with_c=True)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        say("few rows", shape, ta, tb)
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb, check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "few rows %s %s%s" % (shape, ta, tb))
        C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=tb,
                lds=(As.shape[1] + 3, Bs.shape[1] + 1, N + 2), offsets=(1, 3, 2), check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "few rows %s %s%s padded" % (shape, ta, tb))
        Ai, Bi, Ci = draw(M, N, K, seed=M + 5 * N + K, kind="int", with_c=True)
        Ais = np.ascontiguousarray(Ai.T) if ta else Ai
        Bis = np.ascontiguousarray(Bi.T) if tb else Bi
        C = run(Ais, Bis, Ci, 1.0, 1.0, variant=v, trans_a=ta, trans_b=tb)
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "few rows %s %s%s int" % (shape, ta, tb))


@pytest.mark.parametrize("shape", [(4, 16384, 8192), (3, 8201, 16400), (20, 16384, 8192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_rows_matrix_core_kernel_streaming_b(shape):
    """An untransposed B of 512 MiB or more goes through the matrix-core
    few-rows kernel's non-temporal loads: four-column vector loads, one-column
    loads (N odd), two 16-row blocks (M = 20), a padded / misaligned copy;
    real data to 1e-5 and integer data exactly."""
    M, N, K = shape
    assert N * K >= 1 << 27
    v = VNAMES.index("fewrows_m32")
    A, B, Cin = draw(M, N, K, seed=M + N, with_c=True)
    say("few rows streaming B", shape)
    C = run(A, B, Cin, 1.5, 0.5, variant=v, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "few rows streaming %s" % (shape,))
    if M == 4:
        say("few rows streaming B padded", shape)
        C = run(A, B, Cin, 1.5, 0.5, variant=v, lds=(K + 3, N + 1, N + 2), offsets=(1, 3, 2),
                check_outside=True)
        check_real(C, A, B, Cin, 1.5, 0.5, "few rows streaming %s padded" % (shape,))
    del A, B
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + 1, kind="int", with_c=True)
    say("few rows streaming B int", shape)
    C = run(Ai, Bi, Ci, 1.0, 1.0, variant=v)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "few rows streaming %s int" % (shape,))


@pytest.mark.parametrize("shape,ta", [((16, 8192, 8192), False), ((20, 8200, 8193), True),
                                      ((3, 65536, 1024), False)],
                         ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else ("TA" if x else "NA"))
def test_few_rows_matrix_core_kernel_streaming_bt(shape, ta):
    """A transposed B of 256 MiB or more: the waves take batches of K groups
    in turn (the last whole batch, the groups after it and a ragged end on
    the wave next in turn); A as stored or transposed, two 16-row blocks
    (M = 20), one to four column blocks per lane; real data to 1e-5 and
    integer data exactly."""
    M, N, K = shape
    assert N * K >= 1 << 26
    v = VNAMES.index("fewrows_m32")
    A, B, Cin = draw(M, N, K, seed=M + N + 5, with_c=True)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T)
    say("few rows streaming B^T", shape, ta)
    C = run(As, Bs, Cin, 1.5, 0.5, variant=v, trans_a=ta, trans_b=True, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "few rows streaming B^T %s" % (shape,))
    del A, B, Bs
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + 6, kind="int", with_c=True)
    Ais = np.ascontiguousarray(Ai.T) if ta else Ai
    say("few rows streaming B^T int", shape, ta)
    C = run(Ais, np.ascontiguousarray(Bi.T), Ci, 1.0, 1.0, variant=v, trans_a=ta, trans_b=True)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "few rows streaming B^T %s int" % (shape,))


@pytest.mark.parametrize("batch,N", [(16, 1000), (8, 1000), (16, 1001), (3, 130)],
                         ids=lambda x: str(x))
def test_few_rows_matrix_core_kernel_batched(batch, N):
    """Enough slices for the 4- and 2-column lane loads (16 and 8 slices of
    1000 columns), a column count they do not divide (1001), and a small batch
    with one-column loads; B as stored and transposed (4, 2 and 1 column
    blocks per lane); integer data exactly, slices with gaps."""
    rng = np.random.default_rng(batch * 7 + N)
    M, K = (12 if batch % 2 == 0 else 20), 300
    v = VNAMES.index("fewrows_m32")
    Ai = rng.integers(-4, 5, (batch, M, K)).astype(np.float32)
    Bi = rng.integers(-4, 5, (batch, K, N)).astype(np.float32)
    Ci = rng.integers(-4, 5, (batch, M, N)).astype(np.float32)
    say("few rows batched", batch, N)
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=v, gap=3)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, "few rows batch %d N %d" % (batch, N), exact=True)
    # B transposed (stored N x K per slice): the same column-block choice
    Bt = np.ascontiguousarray(np.transpose(Bi, (0, 2, 1)))
    say("few rows batched B^T", batch, N)
    out = run_batched(Ai, Bt, Ci, 1.0, 1.0, variant=v, gap=3, trans_b=True)
    check_batched(out, Ai, Bt, Ci, 1.0, 1.0, "few rows batch %d N %d B^T" % (batch, N), exact=True,
                  tb=True)


@pytest.mark.parametrize("shape", [(4096, 1, 4096), (1000, 7, 3000), (3000, 15, 100), (65536, 8, 1024),
                                   (12, 2500, 777), (8, 4096, 1500), (20, 3000, 1000), (3, 2100, 2500)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_columns_or_rows_automatic(shape):
    """Fewer than 16 columns (or rows) of C through the automatic choice:
    real data to 1e-5, integer data exactly, and a padded / misaligned copy."""
    M, N, K = shape
    A, B, Cin = draw(M, N, K, seed=M + N, with_c=True)
    say("narrow", shape)
    C = run(A, B, Cin, 1.5, 0.5, check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "narrow %s" % (shape,))
    C = run(A, B, Cin, 1.5, 0.5, lds=(K + 1, N + 3, N + 2), offsets=(3, 1, 2), check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "narrow %s padded" % (shape,))
    Ai, Bi, Ci = draw(M, N, K, seed=M + N, kind="int", with_c=True)
    C = run(Ai, Bi, Ci, 1.0, 1.0)
    check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "narrow %s int" % (shape,))


@pytest.mark.parametrize("case", [("auto", (300, 260, 530)), ("mfma32_256x256x32_2x2_sched", (512, 512, 256)),
                                  ("mfma16_64x64x64_4x2_sched_splitk", (64, 64, 4096)),
                                  ("mfma16_64x64x64_4x2_pipe_splitk", (64, 64, 4096)),
                                  ("fewrows_m32", (12, 2048, 1024))], ids=lambda c: c[0])
def test_graph_capture_replays(case):
    """Library calls captured in a HIP graph (through torch's graph capture)
    replay correctly, several times, with eager work in between: every kernel
    the library records is an ordinary launch (split K clears C with its own
    kernel, no memset node).  Integer data, so every replay must equal the
    oracle exactly whatever the order of the split sums."""
    name, (M, N, K) = case
    v = -1 if name == "auto" else VNAMES.index(name)
    Ai, Bi, Ci = draw(M, N, K, seed=M + N + K, kind="int", with_c=True)
    ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (Ai, Bi, Ci))
    out = torch.empty_like(dC0)
    say("graph", name)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up on the capture stream's side
        torch.add(dC0, 0.0, out=out)
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=v)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        torch.add(dC0, 0.0, out=out)  # restore C with a kernel, not a copy node
        sg.gemm(dA, dB, out, 1.0, 1.0, variant=v)
    for i in range(3):
        junk = torch.randn(4096, device="cuda")
        float(junk.abs().sum())       # eager work and a synchronisation between replays
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), "%s replay %d" % (name, i)


def test_runs_on_a_side_stream():
    A, B, _ = draw(512, 384, 256, seed=13)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.full((512, 384), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    say("side stream")
    with torch.cuda.stream(s):
        sg.gemm(dA, dB, dC, 1.0, 0.0)
    s.synchronize()
    check_real(dC.cpu().numpy(), A, B, None, 1.0, 0.0, "side stream")


def test_error_status_raised_from_python():
    dA = torch.zeros((4, 8), device="cuda")
    dB = torch.zeros((8, 4), device="cuda")
    dC = torch.zeros((4, 4), device="cuda")
    with pytest.raises(sg.SgemmError):
        sg.gemm(dA, dB, dC, variant=sg.sgemm_num_variants())
    with pytest.raises(TypeError):
        sg.gemm(dA.double(), dB, dC)


# ---------------------------------------------------------------- full-size workloads

_cache = {}


def _ref(key, fn):
    if key not in _cache:
        _cache[key] = fn()
    return _cache[key]


def test_headline_4096_full_check():
    """M=N=K=4096, alpha=1, beta=0 through the automatic choice; every
    element checked."""
    A, B, _ = draw_workload(HEADLINE)
    say("headline 4096^3 variant", sg.sgemm_variant_name(
        sg.sgemm_select_variant(4096, 4096, 4096, 1.0, 256, 4096, 256, 4096, 0.0, 256, 4096)))
    C = run(A, B)
    err = check_real(C, A, B, None, 1.0, 0.0, "4096^3")
    say("headline normalized error %.3g" % err)


def test_accumulate_4096_full_check_and_integer_copy():
    A, B, Cin = draw_workload(ACCUM)
    say("accumulate 4096^3 real")
    C = run(A, B, Cin, ACCUM.alpha, ACCUM.beta)
    err = check_real(C, A, B, Cin, ACCUM.alpha, ACCUM.beta, "4096^3 accumulate")
    say("accumulate normalized error %.3g" % err)
    Ai, Bi, Ci = draw_workload(ACCUM_INT)
    say("accumulate 4096^3 int")
    C = run(Ai, Bi, Ci, ACCUM_INT.alpha, ACCUM_INT.beta)
    check_exact(C, Ai, Bi, Ci, ACCUM_INT.alpha, ACCUM_INT.beta, "4096^3 accumulate int")
    # dyadic scalars on integer data stay exact too
    C = run(Ai, Bi, Ci, 1.5, 0.5)
    check_exact(C, Ai, Bi, Ci, 1.5, 0.5, "4096^3 int alpha=1.5 beta=0.5")


@pytest.mark.parametrize("w", [w for w in sweep_workloads() if w.M < 8192], ids=lambda w: w.name)
def test_sweep_full_check(w):
    A, B, _ = draw_workload(w)
    say("sweep", w.name)
    C = run(A, B)
    check_real(C, A, B, None, 1.0, 0.0, w.name)
    Ai, Bi, _ = draw(w.M, w.N, w.K, seed=w.seed, kind="int")
    C = run(Ai, Bi)
    check_exact(C, Ai, Bi, None, 1.0, 0.0, w.name + " int")


def _sample(M, N, nrows, ncols, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=min(nrows, M), replace=False))
    cols = np.sort(rng.choice(N, size=min(ncols, N), replace=False))
    return rows, cols


def _sampled_check(A, B, C, alpha, beta, Cin, nrows, ncols, seed, what):
    """Whole rows and whole columns of C (each crosses every tile boundary
    along its length) against the oracle, to the normalized-error bar."""
    M, N = C.shape
    rows, cols = _sample(M, N, nrows, ncols, seed)
    ref, den = oracle.gemm(A, B, Cin, alpha, beta, rows=rows)
    err_r = oracle.normalized_error(C[rows], ref, den)
    ref, den = oracle.gemm(A, B, Cin, alpha, beta, cols=cols)
    err_c = oracle.normalized_error(C[:, cols], ref, den)
    assert max(err_r, err_c) <= TOL, "%s: sampled normalized error %.3g" % (what, max(err_r, err_c))
    return max(err_r, err_c)


def _sampled_exact(A, B, C, alpha, beta, Cin, nrows, ncols, seed, what):
    """Integer data: sampled whole rows and columns equal the oracle exactly."""
    M, N = C.shape
    rows, cols = _sample(M, N, nrows, ncols, seed)
    ref, _ = oracle.gemm(A, B, Cin, alpha, beta, rows=rows)
    assert oracle.exact_match(C[rows], ref), "%s: sampled rows differ from the oracle" % what
    ref, _ = oracle.gemm(A, B, Cin, alpha, beta, cols=cols)
    assert oracle.exact_match(C[:, cols], ref), "%s: sampled columns differ from the oracle" % what


def test_sweep_8192_sampled():
    """8192^3 through the automatic choice: 512 seeded whole rows and 512
    whole columns against the oracle on real data, and the same sample of
    the integer copy exactly (every partial sum is an integer of magnitude
    at most 16 * 8192 < 2^24, so any summation order is exact)."""
    w = [w for w in sweep_workloads() if w.M == 8192][0]
    A, B, _ = draw_workload(w)
    say("sweep 8192^3 real")
    C = run(A, B)
    err = _sampled_check(A, B, C, 1.0, 0.0, None, 512, 512, 8192, w.name)
    say("8192^3 sampled normalized error %.3g" % err)
    del A, B, C
    Ai, Bi, _ = draw(w.M, w.N, w.K, seed=w.seed, kind="int")
    say("sweep 8192^3 int")
    C = run(Ai, Bi)
    _sampled_exact(Ai, Bi, C, 1.0, 0.0, None, 512, 512, 8193, w.name + " int")


@pytest.mark.parametrize("w", ragged_workloads() + shard_workloads(), ids=lambda w: w.name)
def test_rectangular_and_ragged(w):
    A, B, _ = draw_workload(w)
    say("shape", w.name)
    C = run(A, B)
    if w.M * w.N * w.K > 2 ** 36:
        _sampled_check(A, B, C, 1.0, 0.0, None, 256, 256, w.seed, w.name)
    else:
        check_real(C, A, B, None, 1.0, 0.0, w.name)
    Ai, Bi, _ = draw(w.M, w.N, w.K, seed=w.seed, kind="int")
    C = run(Ai, Bi)
    if w.M * w.N * w.K > 2 ** 36:
        rows = np.arange(0, w.M, max(1, w.M // 128))
        ref, _ = oracle.gemm(Ai, Bi, rows=rows)
        assert oracle.exact_match(C[rows], ref), w.name + " int"
    else:
        check_exact(C, Ai, Bi, None, 1.0, 0.0, w.name + " int")


# Shapes whose tile count sits just past whole rounds of the CUs, or whose
# row count sits just past a multiple of 64, where the automatic choice takes
# smaller tiles (32x64, 64x64, 128x64, K split or not); the automatic path,
# with the selection pinned so the intended kernel is the one checked.
TAIL_SHAPES = [((2047, 2049, 2047), "edge_split"),
               ((3000, 3000, 3000), "mfma16_64x64x64_4x2_sched"),
               ((8191, 1025, 8191), "edge_split"),
               ((6144, 1024, 4096), "mfma16_128x64x64_4x2_sched"),
               ((96, 8192, 8192), "mfma16_32x64x64_2x2_sched_splitk"),
               ((160, 4096, 4096), "mfma16_32x64x64_2x2_sched_splitk"),
               ((320, 8192, 8192), "mfma16_32x64x64_2x2_sched"),
               ((32, 8192, 8192), "mfma16_32x64x64_2x2_sched_splitk"),
               ((32, 65536, 1024), "mfma16_32x64x64_2x2_sched")]


@pytest.mark.parametrize("shape,expect", TAIL_SHAPES, ids=lambda v: "x".join(map(str, v))
                         if isinstance(v, tuple) else v)
def test_last_round_tail_shapes(shape, expect):
    M, N, K = shape
    v = sg.sgemm_select_variant(M, N, K, 1.0, 1, K, 1, N, 0.0, 1, N)
    assert sg.sgemm_variant_name(v) == expect
    A, B, _ = draw(M, N, K, seed=M + N + K)
    say("tail shape", shape, expect)
    C = run(A, B)
    _sampled_check(A, B, C, 1.0, 0.0, None, 192, 192, M, "tail %s" % (shape,))
    Ai, Bi, _ = draw(M, N, K, seed=M + N + K, kind="int")
    C = run(Ai, Bi)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 96)), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 96)), [N - 1]]))
    ref, _ = oracle.gemm(Ai, Bi, rows=rows)
    assert oracle.exact_match(C[rows], ref), "tail %s int rows" % (shape,)
    ref, _ = oracle.gemm(Ai, Bi, cols=cols)
    assert oracle.exact_match(C[:, cols], ref), "tail %s int cols" % (shape,)


# The edge split: a thin edge of 1 to 16 columns (or rows) split off to the
# few-columns (few-rows) kernel, the bulk on whole rounds of large tiles.
EDGE_SHAPES = [((4095, 4097, 1023), "NN"), ((4095, 4097, 1023), "NT"), ((4095, 4097, 1023), "TN"),
               ((4095, 4097, 1023), "TT"), ((4097, 4097, 4097), "NN"), ((1025, 1024, 1024), "NN"),
               ((1025, 1024, 1024), "TT"), ((2047, 2049, 2047), "NT"),
               # column edges of 32 and 24: two few-columns strips (16, then the rest)
               ((2048, 2080, 2048), "NN"), ((4096, 4120, 2048), "TN")]


@pytest.mark.parametrize("shape,ops", EDGE_SHAPES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple)
                         else v)
def test_edge_split_automatic(shape, ops):
    """The automatic choice takes the edge split (both edges at (4097, 4097,
    4097); a one-row edge at (1025, 1024, 1024); column edges of 24 and 32 in
    two strips), in every orientation, with
    alpha and beta: whole rows and columns of real data to 1e-5 (every
    element for the smaller shapes), and integer data exactly."""
    M, N, K = shape
    ta, tb = ops[0] == "T", ops[1] == "T"
    lda, ldb = (M if ta else K), (K if tb else N)
    v = sg.sgemm_strided_batched_select_variant(int(ta), int(tb), M, N, K, 1.0, 256, lda, 0, 256, ldb, 0,
                                                0.5, 256, N, 0, 1)
    assert sg.sgemm_variant_name(v) == "edge_split", sg.sgemm_variant_name(v)
    A, B, Cin = draw(M, N, K, seed=M + 2 * N + K, with_c=True)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    say("edge split", shape, ops)
    C = run(As, Bs, Cin, 1.5, 0.5, trans_a=ta, trans_b=tb, check_outside=True)
    if M * N * K > 2 ** 32:
        _sampled_check(A, B, C, 1.5, 0.5, Cin, 160, 160, M, "edge split %s %s" % (shape, ops))
        # the thin edge itself, whole
        ref, den = oracle.gemm(A, B, Cin, 1.5, 0.5, cols=np.arange(N - N % 64, N))
        assert oracle.normalized_error(C[:, N - N % 64:], ref, den) <= TOL
    else:
        check_real(C, A, B, Cin, 1.5, 0.5, "edge split %s %s" % (shape, ops))
    Ai, Bi, Ci = draw(M, N, K, seed=M + 2 * N + K + 1, kind="int", with_c=True)
    Ais = np.ascontiguousarray(Ai.T) if ta else Ai
    Bis = np.ascontiguousarray(Bi.T) if tb else Bi
    C = run(Ais, Bis, Ci, 1.0, 1.0, trans_a=ta, trans_b=tb)
    if M * N * K > 2 ** 32:
        rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 96)), np.arange(M - M % 64, M)]))
        cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 96)), np.arange(N - N % 64, N)]))
        ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0, rows=rows)
        assert oracle.exact_match(C[rows], ref), "edge split %s %s int rows" % (shape, ops)
        ref, _ = oracle.gemm(Ai, Bi, Ci, 1.0, 1.0, cols=cols)
        assert oracle.exact_match(C[:, cols], ref), "edge split %s %s int cols" % (shape, ops)
    else:
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "edge split %s %s int" % (shape, ops))


# Shapes the automatic choice gives the edge split, drawn once with a seeded
# generator over M, N = (4..24) x (64, 128 or 256) + (1..16 or 0), K 1000-2600
# and every orientation.
EDGE_RANDOM = [(1293, 6152, 1114, "NT"), (1024, 5122, 1438, "TT"), (2947, 2825, 2373, "NT"),
               (6144, 6154, 1999, "TN"), (3072, 4105, 1229, "NN"), (5387, 3854, 2393, "NN"),
               (2053, 5888, 1615, "TN"), (4864, 2572, 2592, "NN"), (4864, 3333, 2311, "NN"),
               (4610, 1798, 1047, "NN")]


@pytest.mark.parametrize("case", EDGE_RANDOM, ids=lambda c: "%dx%dx%d-%s" % c)
def test_edge_split_random_shapes(case):
    """Integer data exactly on sampled rows and columns, the edges whole."""
    M, N, K, ops = case
    ta, tb = ops[0] == "T", ops[1] == "T"
    v = sg.sgemm_strided_batched_select_variant(int(ta), int(tb), M, N, K, 1.0, 256, M if ta else K, 0, 256,
                                                K if tb else N, 0, 0.0, 256, N, 0, 1)
    assert sg.sgemm_variant_name(v) == "edge_split"
    Ai, Bi, _ = draw(M, N, K, seed=M * 7 + N + K, kind="int")
    Ais = np.ascontiguousarray(Ai.T) if ta else Ai
    Bis = np.ascontiguousarray(Bi.T) if tb else Bi
    say("edge split random", case)
    C = run(Ais, Bis, trans_a=ta, trans_b=tb, check_outside=True)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 48)), np.arange(M - M % 64, M), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 48)), np.arange(N - N % 64, N), [N - 1]]))
    ref, _ = oracle.gemm(Ai, Bi, rows=rows)
    assert oracle.exact_match(C[rows], ref), "%s rows" % (case,)
    ref, _ = oracle.gemm(Ai, Bi, cols=cols)
    assert oracle.exact_match(C[:, cols], ref), "%s cols" % (case,)


def test_edge_split_padded_batched_and_workspace():
    """The edge split forced on padded, misaligned operands (nothing outside C
    written); over a strided batch with gaps between the slices; and through
    the workspace entry point, whose choice it is as well."""
    v = VNAMES.index("edge_split")
    M, N, K = 1031, 1030, 1100
    A, B, Cin = draw(M, N, K, seed=77, with_c=True)
    say("edge split padded")
    C = run(A, B, Cin, 1.5, 0.5, variant=v, lds=(K + 3, N + 1, N + 5), offsets=(1, 3, 2), check_outside=True)
    check_real(C, A, B, Cin, 1.5, 0.5, "edge split padded")
    rng = np.random.default_rng(78)
    batch, M, N, K = 3, 1025, 1024, 1024
    Ai = rng.integers(-4, 5, (batch, M, K)).astype(np.float32)
    Bi = rng.integers(-4, 5, (batch, K, N)).astype(np.float32)
    Ci = rng.integers(-4, 5, (batch, M, N)).astype(np.float32)
    say("edge split batched")
    out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=v, gap=3)
    check_batched(out, Ai, Bi, Ci, 1.0, 1.0, "edge split batched", exact=True)
    M, N, K = 4095, 4097, 1023
    ws = torch.zeros(4096 + (32 << 20), dtype=torch.uint8, device="cuda")
    w = sg.sgemm_strided_batched_ws_select_variant(0, 0, M, N, K, 1.0, 256, K, 0, 256, N, 0, 0.0, 256, N, 0, 1,
                                                   ws.numel())
    assert sg.sgemm_variant_name(w) == "edge_split"
    Ai, Bi, _ = draw(M, N, K, seed=79, kind="int")
    say("edge split workspace")
    C = run(Ai, Bi, workspace=ws)
    cols = np.unique(np.concatenate([np.arange(0, N, 61), np.arange(N - 64, N)]))
    ref, _ = oracle.gemm(Ai, Bi, cols=cols)
    assert oracle.exact_match(C[:, cols], ref)
    assert bool((ws[:4096] == 0).all().item())


# Shapes whose default choice adds partial sums with atomics: K-split tiles
# (few tiles, long K) and the split form of the vector-unit few-rows kernel.
ATOMIC_SHAPES = [(64, 8192, 8192), (96, 8192, 8192), (8, 512, 4096), (300, 40, 100000)]


@pytest.mark.parametrize("shape", ATOMIC_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_atomics_not_allowed_repeatable(shape):
    """With atomics not allowed, the automatic choice leaves the atomic forms
    and two calls on the same inputs give bitwise the same C, within the
    tolerance of the oracle."""
    M, N, K = shape
    default = sg.sgemm_variant_name(sg.sgemm_select_variant(M, N, K, 1.0, 1, K, 1, N, 0.0, 1, N))
    assert default.endswith("_splitk") or default == "skinny_m8", default
    A, B, _ = draw(M, N, K, seed=7 + M)
    try:
        assert sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_NOT_ALLOWED) == sg.SGEMM_OK
        name = sg.sgemm_variant_name(sg.sgemm_select_variant(M, N, K, 1.0, 1, K, 1, N, 0.0, 1, N))
        assert not name.endswith("_splitk") and name != "skinny_m8", name
        say("no atomics", shape, name)
        C1 = run(A, B)
        C2 = run(A, B)
    finally:
        sg.sgemm_set_atomics_mode(sg.SGEMM_ATOMICS_ALLOWED)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "%s: repeated calls differ" % (shape,)
    if M * N * K > 2 ** 32:
        _sampled_check(A, B, C1, 1.0, 0.0, None, 128, 128, M, "no atomics %s" % (shape,))
    else:
        check_real(C1, A, B, None, 1.0, 0.0, "no atomics %s" % (shape,))
    say("atomics", shape, default)
    C3 = run(A, B)
    if M * N * K > 2 ** 32:
        _sampled_check(A, B, C3, 1.0, 0.0, None, 128, 128, M, "atomics %s" % (shape,))
    else:
        check_real(C3, A, B, None, 1.0, 0.0, "atomics %s" % (shape,))


R32 = [v for v in VARIANTS if VNAMES[v].startswith("mfma16_32x64x64")]


@pytest.mark.parametrize("variant", R32, ids=[VNAMES[v] for v in R32])
@pytest.mark.parametrize("ops", [(False, False), (False, True), (True, False)], ids=["NN", "NT", "TN"])
def test_rows32_fewer_rows_than_the_tile(variant, ops):
    """The 32-row tiles with M below 32 (A untransposed: rows past M read row
    M - 1 and are never stored; A transposed: the fallback), with padded and
    misaligned operands, K split or not: exact on integer data, nothing
    outside C written, and the accumulate form on real data."""
    ta, tb = ops
    for (M, N, K) in [(1, 64, 64), (2, 65, 300), (15, 130, 64), (17, 333, 1000), (24, 256, 8192),
                      (31, 200, 129), (31, 64, 4096)]:
        Ai, Bi, Ci = draw(M, N, K, seed=5 * M + N + K, kind="int", with_c=True)
        A = np.ascontiguousarray(Ai.T) if ta else Ai
        B = np.ascontiguousarray(Bi.T) if tb else Bi
        lds = (A.shape[1] + 3, B.shape[1] + 5, N + 7)
        say("rows32", VNAMES[variant], ops, (M, N, K))
        C = run(A, B, Ci, 1.0, 1.0, variant=variant, trans_a=ta, trans_b=tb, lds=lds,
                offsets=(1, 2, 3), check_outside=True)
        check_exact(C, Ai, Bi, Ci, 1.0, 1.0, "%s %s (%d,%d,%d)" % (VNAMES[variant], ops, M, N, K))
        Ar, Br, Cr = draw(M, N, K, seed=7 * M + N + K, with_c=True)
        A = np.ascontiguousarray(Ar.T) if ta else Ar
        B = np.ascontiguousarray(Br.T) if tb else Br
        C = run(A, B, Cr, 1.5, 0.5, variant=variant, trans_a=ta, trans_b=tb, check_outside=True)
        check_real(C, Ar, Br, Cr, 1.5, 0.5, "%s %s (%d,%d,%d) real" % (VNAMES[variant], ops, M, N, K))


@pytest.mark.parametrize("variant", R32 + [-1], ids=[VNAMES[v] for v in R32] + ["automatic"])
def test_rows32_fewer_rows_batched(variant):
    """Strided batches with M below the 32-row tile, B untransposed and
    transposed, slices with gaps: real data to the tolerance and integer data
    exactly (the automatic choice takes the 32-row split tiles for the large
    case: 20 rows, N*K*batch >= 2^25)."""
    rng = np.random.default_rng(43)
    for tb in (False, True):
        for (batch, M, N, K) in ((3, 20, 130, 300), (4, 20, 1024, 8192)):
            A = rng.uniform(-1, 1, (batch, M, K)).astype(np.float32)
            B = rng.uniform(-1, 1, (batch, N, K) if tb else (batch, K, N)).astype(np.float32)
            C = rng.standard_normal((batch, M, N)).astype(np.float32)
            say("rows32 batched", variant, tb, (batch, M, N, K))
            out = run_batched(A, B, C, 1.5, 0.5, variant=variant, trans_b=tb, gap=5)
            check_batched(out, A, B, C, 1.5, 0.5, "rows32 batched %s" % variant, tb=tb)
            Ai = rng.integers(-4, 5, A.shape).astype(np.float32)
            Bi = rng.integers(-4, 5, B.shape).astype(np.float32)
            Ci = rng.integers(-4, 5, C.shape).astype(np.float32)
            out = run_batched(Ai, Bi, Ci, 1.0, 1.0, variant=variant, trans_b=tb)
            check_batched(out, Ai, Bi, Ci, 1.0, 1.0, "rows32 batched int %s" % variant, exact=True, tb=tb)
