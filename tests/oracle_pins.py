"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin takes a loaded oracle library and raises AssertionError when the oracle
disagrees with something the mathematics or the pages fix:
  * closed forms: identity and permutation matrices, all-ones, integer rank-1 products;
  * invariants that hold exactly on small integers: the transpose identity and
    additivity over a split of K;
  * an exact brute force in Python integers / rationals on the pages' tiny worked shapes
    (6 x 6 x 9 from "SGEMM: Shared Memory Tiling Visualizer", controls; 4 x 8 times 8 x 4
    from the same page's memory panels; 8 x 8 times 8 x 8 from "SGEMM: 2D Register Tiling
    Visualizer", memory panels), which is a different code path from the C loop;
  * the fp64 rounding bound against the exact rational result;
  * numpy's float64 matmul (a library routine) within fp64 rounding.
Every pin is run against the real oracle in test_oracle_pins.py, and against
deliberately broken copies of it in test_oracle_mutations.py, which checks that each
plausible mistake (dropped term, wrong sign, swapped index, wrong stride) trips a pin.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle

U = 2.0 ** -53  # unit roundoff of IEEE double


def _ints(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def _exact_int_product(A: np.ndarray, B: np.ndarray) -> list[list[int]]:
    """Row-by-column sums in Python integers (no floating point anywhere)."""
    Ai = [[int(v) for v in row] for row in A]
    Bi = [[int(v) for v in row] for row in B]
    M, K, N = len(Ai), len(Bi), len(Bi[0]) if Bi else 0
    return [[sum(Ai[i][k] * Bi[k][j] for k in range(K)) for j in range(N)] for i in range(M)]


def _exact_rational_product(A: np.ndarray, B: np.ndarray):
    """Exact products and magnitude sums of float32 inputs, in rationals."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    ref = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
           for i in range(M)]
    den = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
           for i in range(M)]
    return ref, den


# ----------------------------------------------------------------------------- pins -------

def pin_identity(lib):
    """I_K x B == B bit for bit, for float B and a rectangular K x N."""
    rng = np.random.default_rng(11)
    K, N = 37, 23
    B = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
    eye = np.eye(K, dtype=np.float32)
    C = oracle.gemm_f64(eye, B, lib=lib)
    assert np.array_equal(C, B.astype(np.float64)), "I x B != B"
    # and on the other side: A x I_K == A
    A = rng.uniform(-1, 1, size=(19, K)).astype(np.float32)
    C2 = oracle.gemm_f64(A, eye, lib=lib)
    assert np.array_equal(C2, A.astype(np.float64)), "A x I != A"


def pin_permutation(lib):
    """P x B == B[perm] and B x P' permutes columns, bit for bit."""
    rng = np.random.default_rng(12)
    K, N = 29, 31
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[np.arange(K), perm] = 1.0
    B = rng.standard_normal(size=(K, N)).astype(np.float32)
    C = oracle.gemm_f64(P, B, lib=lib)
    assert np.array_equal(C, B[perm].astype(np.float64)), "P x B != B[perm]"
    permc = rng.permutation(N)
    Q = np.zeros((N, N), dtype=np.float32)
    Q[permc, np.arange(N)] = 1.0
    C2 = oracle.gemm_f64(B, Q, lib=lib)
    assert np.array_equal(C2, B[:, permc].astype(np.float64)), "B x Q != B[:, perm]"


def pin_all_ones(lib):
    """ones(M,K) x ones(K,N) == K everywhere."""
    for (M, N, K) in [(3, 5, 7), (6, 6, 9), (1, 1, 1), (4, 4, 8)]:
        C = oracle.gemm_f64(np.ones((M, K), np.float32), np.ones((K, N), np.float32), lib=lib)
        assert np.all(C == K), f"ones product != {K} at {M}x{N}x{K}"


def pin_rank_one(lib):
    """(u v^T)(x y^T) == (v . x) u y^T on integers (exact in both precisions)."""
    rng = np.random.default_rng(13)
    M, K, N = 7, 11, 5
    u, v = rng.integers(-3, 4, M), rng.integers(-3, 4, K)
    x, y = rng.integers(-3, 4, K), rng.integers(-3, 4, N)
    A = np.outer(u, v).astype(np.float32)
    B = np.outer(x, y).astype(np.float32)
    expect = int(np.dot(v, x)) * np.outer(u, y)
    C = oracle.gemm_f64(A, B, lib=lib)
    assert np.array_equal(C, expect.astype(np.float64)), "rank-1 closed form"


def pin_worked_shapes_exact(lib):
    """Small-integer matrices at the pages' tiny shapes against Python-integer sums."""
    rng = np.random.default_rng(14)
    for (M, N, K) in [(6, 6, 9), (4, 4, 8), (8, 8, 8), (1, 7, 3), (5, 2, 1)]:
        A = _ints(rng, (M, K))
        B = _ints(rng, (K, N))
        exact = np.array(_exact_int_product(A, B), dtype=np.float64)
        C = oracle.gemm_f64(A, B, lib=lib)
        assert np.array_equal(C, exact), f"integer brute force differs at {M}x{N}x{K}"


def pin_transpose_identity(lib):
    """(A B)^T == B^T A^T, exactly on integers."""
    rng = np.random.default_rng(15)
    A = _ints(rng, (9, 13))
    B = _ints(rng, (13, 6))
    C = oracle.gemm_f64(A, B, lib=lib)
    Ct = oracle.gemm_f64(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), lib=lib)
    assert np.array_equal(C.T, Ct), "(AB)^T != B^T A^T"


def pin_k_split(lib):
    """A B == A[:, :k1] B[:k1] + A[:, k1:] B[k1:], exactly on integers."""
    rng = np.random.default_rng(16)
    M, N, K, k1 = 8, 10, 17, 6
    A = _ints(rng, (M, K))
    B = _ints(rng, (K, N))
    C = oracle.gemm_f64(A, B, lib=lib)
    C1 = oracle.gemm_f64(np.ascontiguousarray(A[:, :k1]), np.ascontiguousarray(B[:k1]), lib=lib)
    C2 = oracle.gemm_f64(np.ascontiguousarray(A[:, k1:]), np.ascontiguousarray(B[k1:]), lib=lib)
    assert np.array_equal(C, C1 + C2), "K-split additivity"


def pin_rational_bound(lib):
    """Float inputs at the worked shapes: |C - exact| <= (K-1) u den (fp64 sum bound)."""
    rng = np.random.default_rng(17)
    for (M, N, K) in [(6, 6, 9), (4, 4, 8), (8, 8, 8), (3, 4, 33)]:
        A = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
        B = rng.standard_normal(size=(K, N)).astype(np.float32)
        ref, den = _exact_rational_product(A, B)
        C = oracle.gemm_f64(A, B, lib=lib)
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(float(C[i, j])) - ref[i][j])
                bound = Fraction(max(K - 1, 1)) * Fraction(U) * den[i][j]
                assert err <= bound, f"fp64 bound violated at ({i},{j}) of {M}x{N}x{K}"


def pin_numpy_matmul(lib):
    """Against numpy's float64 matmul on a ragged shape, within the fp64 sum bound."""
    rng = np.random.default_rng(18)
    M, N, K = 33, 47, 129
    A = rng.standard_normal(size=(M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    den = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    C = oracle.gemm_f64(A, B, lib=lib)
    assert np.all(np.abs(C - ref) <= 2 * K * U * den + 1e-300), "differs from numpy matmul"


def pin_leading_dimensions(lib):
    """Operands embedded in wider NaN-padded arrays give the packed result bit for bit."""
    rng = np.random.default_rng(19)
    M, N, K = 5, 7, 9
    A = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
    Abuf = np.full((M, K + 3), np.nan, np.float32)
    Abuf[:, :K] = A
    Bbuf = np.full((K, N + 5), np.nan, np.float32)
    Bbuf[:, :N] = B
    C = oracle.gemm_f64(A, B, lib=lib)
    Cv = oracle.gemm_f64(Abuf[:, :K], Bbuf[:, :N], lib=lib)
    assert np.array_equal(C, Cv), "leading dimensions change the result"
    assert np.all(np.isfinite(Cv)), "padding leaked into the product"


def pin_check_exact(lib):
    """oracle.check reports zero error for the exact answer of a closed form, and the
    exact normalised error of a planted perturbation at its location."""
    M, N, K = 6, 6, 9
    rng = np.random.default_rng(20)
    A = np.ones((M, K), np.float32)
    B = _ints(rng, (K, N), -2, 2)
    exact = np.tile(B.sum(axis=0), (M, 1)).astype(np.float32)   # column sums, exact
    den = np.tile(np.abs(B).sum(axis=0), (M, 1)).astype(np.float64)
    rep = oracle.check(A, B, exact, lib=lib)
    assert rep["n_inexact"] == 0 and rep["max_err"] == 0.0 and rep["n_checked"] == M * N, rep
    assert rep["n_nonfinite"] == 0 and rep["n_zero_den_bad"] == 0, rep
    j = int(np.argmax(den[2]))
    bad = exact.copy()
    bad[2, j] += 0.5
    rep = oracle.check(A, B, bad, lib=lib)
    assert rep["n_inexact"] == 1 and (rep["arg_i"], rep["arg_j"]) == (2, j), rep
    assert rep["max_err"] == 0.5 / den[2, j], rep
    bad2 = exact.copy()
    bad2[4, 1] = np.nan
    rep = oracle.check(A, B, bad2, rows=[4], lib=lib)
    assert rep["n_nonfinite"] == 1 and rep["n_checked"] == N, rep
    # zero denominator: a zero row of A forces C's row to be exactly zero
    Az = A.copy()
    Az[3] = 0
    ez = exact.copy()
    ez[3] = 0
    assert oracle.check(Az, B, ez, lib=lib)["n_zero_den_bad"] == 0
    ez[3, 0] = 1e-30
    assert oracle.check(Az, B, ez, lib=lib)["n_zero_den_bad"] == 1


def pin_check_integer(lib):
    """oracle.check on non-constant small-integer A and B at the pages' worked shapes and
    at square shapes (M = N = K, where a transposed or mis-strided operand index still
    reads inside the arrays): the exact answer, from Python-integer sums, must be reported
    exact everywhere, and an error planted at any one position must be reported there,
    with the exact normalised size 1 / sum_k |a_ik b_kj|.
    Each C element is the length-K dot product of row i of A with column j of B ("SGEMM:
    Shared Memory Tiling Visualizer", "Why Tiling Works (The Math)")."""
    rng = np.random.default_rng(23)
    shapes = [(7, 7, 7), (9, 9, 9), (6, 6, 9), (4, 4, 8), (8, 8, 8), (5, 11, 3)]
    for (M, N, K) in shapes:
        A = _ints(rng, (M, K))
        B = _ints(rng, (K, N))
        # no zero rows of A or columns of B, so every magnitude sum is positive
        A[A == 0] = 1
        B[B == 0] = -1
        exact_i = _exact_int_product(A, B)
        den_i = [[sum(abs(int(A[i, k]) * int(B[k, j])) for k in range(K)) for j in range(N)]
                 for i in range(M)]
        exact = np.array(exact_i, dtype=np.float32)
        rep = oracle.check(A, B, exact, lib=lib)
        assert rep["n_checked"] == M * N, rep
        assert rep["n_inexact"] == 0 and rep["max_err"] == 0.0, (M, N, K, rep)
        assert rep["n_nonfinite"] == 0 and rep["n_zero_den_bad"] == 0, rep
        for (i, j) in [(0, 0), (M - 1, N - 1), (M // 2, N - 1), (M - 1, 0), (M // 3, N // 2)]:
            bad = exact.copy()
            bad[i, j] += 1.0
            rep = oracle.check(A, B, bad, lib=lib)
            assert rep["n_inexact"] == 1, (M, N, K, i, j, rep)
            assert (rep["arg_i"], rep["arg_j"]) == (i, j), (M, N, K, i, j, rep)
            assert rep["max_err"] == 1.0 / den_i[i][j], (M, N, K, i, j, rep)
            # the same row checked alone, and a row list that skips it
            rep = oracle.check(A, B, bad, rows=[i], lib=lib)
            assert rep["n_checked"] == N and rep["n_inexact"] == 1, rep
            others = [r for r in range(M) if r != i]
            rep = oracle.check(A, B, bad, rows=others, lib=lib)
            assert rep["n_inexact"] == 0 and rep["n_checked"] == (M - 1) * N, rep


def pin_sample_integer(lib):
    """oracle.sample on non-constant small-integer A and B at square and worked shapes:
    every element against Python-integer sums, and every magnitude sum against
    sum_k |a_ik b_kj| in integers."""
    rng = np.random.default_rng(24)
    for (M, N, K) in [(8, 8, 8), (6, 6, 9), (5, 9, 4)]:
        A = _ints(rng, (M, K))
        B = _ints(rng, (K, N))
        exact = np.array(_exact_int_product(A, B), dtype=np.float64)
        den = np.array([[sum(abs(int(A[i, k]) * int(B[k, j])) for k in range(K))
                         for j in range(N)] for i in range(M)], dtype=np.float64)
        iv, jv = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ref, d = oracle.sample(A, B, iv.ravel(), jv.ravel(), lib=lib)
        assert np.array_equal(ref, exact.ravel()), f"sample values at {M}x{N}x{K}"
        assert np.array_equal(d, den.ravel()), f"sample magnitude sums at {M}x{N}x{K}"


def pin_sample(lib):
    """oracle.sample on closed forms: identity (value and |value| as magnitude sum),
    all-ones (K and K)."""
    rng = np.random.default_rng(21)
    K, N = 12, 9
    B = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
    ii = rng.integers(0, K, 20)
    jj = rng.integers(0, N, 20)
    ref, den = oracle.sample(np.eye(K, dtype=np.float32), B, ii, jj, lib=lib)
    assert np.array_equal(ref, B[ii, jj].astype(np.float64)), "sample on identity"
    assert np.array_equal(den, np.abs(B[ii, jj]).astype(np.float64)), "sample magnitude"
    ref, den = oracle.sample(np.ones((3, 7), np.float32), np.ones((7, 4), np.float32),
                             [0, 2, 1], [3, 0, 2], lib=lib)
    assert np.all(ref == 7) and np.all(den == 7), "sample on ones"
    A = _ints(rng, (6, 9))
    Bi = _ints(rng, (9, 6))
    exact = np.array(_exact_int_product(A, Bi), dtype=np.float64)
    iv, jv = np.meshgrid(np.arange(6), np.arange(6), indexing="ij")
    ref, _ = oracle.sample(A, Bi, iv.ravel(), jv.ravel(), lib=lib)
    assert np.array_equal(ref, exact.ravel()), "sample on integer brute force"


def pin_transpose(lib):
    """The transpose oracle: a hand-written 2 x 3 case, involution, and (AB)^T = B^T A^T
    through the GEMM oracle on integers."""
    X = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    assert np.array_equal(oracle.transpose(X, lib=lib), np.array([[1, 4], [2, 5], [3, 6]], np.float32))
    rng = np.random.default_rng(22)
    Y = rng.standard_normal((37, 19)).astype(np.float32)
    assert np.array_equal(oracle.transpose(oracle.transpose(Y, lib=lib), lib=lib), Y)
    A = _ints(rng, (5, 7))
    B = _ints(rng, (7, 4))
    AB = oracle.gemm_f64(A, B, lib=lib).astype(np.float32)
    BtAt = oracle.gemm_f64(oracle.transpose(B, lib=lib), oracle.transpose(A, lib=lib), lib=lib)
    assert np.array_equal(oracle.transpose(AB, lib=lib), BtAt.astype(np.float32))
    Z = np.full((3, 8), np.nan, np.float32)
    Z[:, :5] = 1
    assert np.array_equal(oracle.transpose(Z[:, :5], lib=lib), np.ones((5, 3), np.float32))


ALL_PINS = [pin_identity, pin_permutation, pin_all_ones, pin_rank_one,
            pin_worked_shapes_exact, pin_transpose_identity, pin_k_split,
            pin_rational_bound, pin_numpy_matmul, pin_leading_dimensions,
            pin_check_exact, pin_check_integer, pin_sample, pin_sample_integer,
            pin_transpose]
