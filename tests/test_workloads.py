"""CPU tests: the seeded input generators are deterministic and as described."""
import numpy as np

from workloads import (ACCUM, ACCUM_INT, HEADLINE, SMALL, SMALL_INT, draw,
                       draw_workload, offset_view, padded, ragged_workloads,
                       sweep_workloads)


def test_draw_is_deterministic_and_shaped():
    a1, b1, c1 = draw(5, 7, 3, seed=42, with_c=True)
    a2, b2, c2 = draw(5, 7, 3, seed=42, with_c=True)
    assert a1.shape == (5, 3) and b1.shape == (3, 7) and c1.shape == (5, 7)
    assert all(x.dtype == np.float32 and x.flags.c_contiguous for x in (a1, b1, c1))
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2) and np.array_equal(c1, c2)
    a3, _, _ = draw(5, 7, 3, seed=43)
    assert not np.array_equal(a1, a3)


def test_value_ranges():
    a, b, c = draw(300, 300, 300, seed=0, with_c=True)
    assert a.min() >= -1 and a.max() <= 1 and b.min() >= -1 and b.max() <= 1
    assert abs(float(c.mean())) < 0.05 and 0.9 < float(c.std()) < 1.1
    assert not np.array_equal(a, b.T)
    ai, bi, ci = draw(300, 300, 300, seed=0, kind="int", with_c=True)
    for x in (ai, bi, ci):
        assert set(np.unique(x).tolist()) == set(range(-4, 5))


def test_named_workloads():
    assert (SMALL.M, SMALL.N, SMALL.K, SMALL.alpha, SMALL.beta) == (256, 256, 256, 1.0, 0.0)
    assert SMALL_INT.kind == "int"
    assert (HEADLINE.M, HEADLINE.beta) == (4096, 0.0)
    assert (ACCUM.alpha, ACCUM.beta) == (1.5, 0.5)
    assert (ACCUM_INT.alpha, ACCUM_INT.beta, ACCUM_INT.kind) == (1.0, 1.0, "int")
    assert [w.M for w in sweep_workloads()] == [128, 256, 512, 1024, 2048, 4096, 8192]
    shapes = [(w.M, w.N, w.K) for w in ragged_workloads()]
    assert (127, 129, 17) in shapes and (1, 4096, 4096) in shapes
    a, b, c = draw_workload(SMALL)
    assert c is None and a.shape == (256, 256)


def test_padded_and_offset_views():
    x = np.arange(12, dtype=np.float32).reshape(3, 4)
    p = padded(x, 7)
    assert p.strides == (28, 4) and np.array_equal(p, x)
    assert np.isnan(p.base[:, 4:]).all()
    o = offset_view(x, 1, ld=5)
    assert np.array_equal(o, x) and o.ctypes.data % 16 == 4 and o.strides == (20, 4)
