"""The seeded operand generators: shapes, distributions, determinism, padding."""
import numpy as np
import pytest

import workloads as wl


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_shapes_and_determinism(name):
    w = wl.WORKLOADS[name]
    A, B = wl.operands(name)
    A2, B2 = wl.operands(name)
    assert A.shape == (w.M, w.K) and B.shape == (w.K, w.N)
    assert A.dtype == np.float32 and A.flags.c_contiguous
    assert np.array_equal(A, A2) and np.array_equal(B, B2)
    if w.dist == "uniform":
        assert A.min() >= -1 and A.max() <= 1
    Ai, Bi = wl.operands(name, "int")
    assert set(np.unique(Ai)).issubset(set(range(-4, 5)))
    assert not np.array_equal(A, Ai[: A.shape[0], : A.shape[1]])


def test_normal_moments():
    A, _ = wl.operands("c3")
    assert abs(A.mean()) < 0.01 and abs(A.std() - 1) < 0.01


def test_padded_views_poisoned():
    A, B = wl.random_operands(5, 7, 9, seed=3, lda=12, ldb=8)
    assert A.strides[0] == 12 * 4 and B.strides[0] == 8 * 4
    assert np.isnan(A.base[:, 9:]).all() and np.isnan(B.base[:, 7:]).all()
    assert np.isfinite(A).all() and np.isfinite(B).all()
