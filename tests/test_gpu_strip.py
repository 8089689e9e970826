"""The column strip through the C ABI: when N leaves one column past the last whole tile
column, the workgroups of the last tile column also compute that column, on the vector
ALUs between their MFMAs, from the A operands they read for the MFMAs. Checked
against the oracle (exact on small integers, within the normalised tolerance on floats)
with NaN-poisoned row padding and guard bands around C, for every strip-capable variant
forced, for the automatic plan, and for run-to-run determinism."""
import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl
from gpu_util import TOL, GuardedC, device_matrix, run_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return torch


def strip_variants():
    return [v for v in range(len(g.variant_names())) if g.sgemm_f32_variant_info(v)["strip"]]


def shapes_for(v):
    """(M, N, K) with N = (whole tile columns) + 1: enough tile columns that every tile takes
    a share of the strip's rows (five or more; 17 gives shares that end inside the tiles),
    K on both sides of the panel depth and of K-group rounds (with partial last panels),
    M ragged; and two products without a strip (a wider remainder, too few tile columns)."""
    bn = g.sgemm_f32_variant_info(v)["BN"]
    return [(63, 5 * bn + 1, 33), (130, 8 * bn + 1, 256), (200, 5 * bn + 1, 257),
            (65, 17 * bn + 1, 300), (257, 5 * bn + 1, 5), (129, 6 * bn + 1, 1),
            (70, 5 * bn + 1, 2050), (17, 9 * bn + 1, 4353), (100, 5 * bn + 1, 37),
            (33, 7 * bn + 1, 64),
            # no strip: a remainder wider than it, or too few tile columns to share its rows
            (130, 5 * bn + 2, 256), (65, bn + 1, 300)]


def _check(A, B, C, kind, what):
    rep = oracle.check(A, B, C)
    assert rep["n_nonfinite"] == 0, (what, rep)
    if kind == "int":
        assert rep["n_inexact"] == 0, (what, rep)
    else:
        assert rep["max_err"] <= TOL, (what, rep)


def test_strip_variants_exist():
    vs = strip_variants()
    assert vs, "no variant computes a column strip"
    for v in vs:
        info = g.sgemm_f32_variant_info(v)
        assert info["direct_loads"] and info["kernel"] == "mfma", info


def test_strip_shapes_forced(gpu):
    for v in strip_variants():
        _strip_shapes(gpu, v)


def _strip_shapes(gpu, v):
    name = g.variant_names()[v]
    for (M, N, K) in shapes_for(v):
        rng = np.random.default_rng(M * 7919 + N * 31 + K)
        A = wl.draw(rng, (M, K), "int")
        B = wl.draw(rng, (K, N), "int")
        for lda, ldb, ldc in [(K + 3, N + 5, N + 2), (K, N, N)]:
            _, dA, _ = device_matrix(A, lda)
            _, dB, _ = device_matrix(B, ldb)
            c = GuardedC(M, N, ldc)
            print(f"[strip] {name} {M}x{N}x{K} lda={lda} ldb={ldb} ldc={ldc}", flush=True)
            run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
            gpu.cuda.synchronize()
            _check(A, B, c.result(), "int", (name, M, N, K, lda, ldb, ldc))


@pytest.mark.parametrize("kind", ["int", "float"])
def test_ragged_workload_plan_uses_strip(gpu, kind):
    """The ragged 1023 x 1025 x 1027 workload: the plan puts its last column in a strip, and
    the result matches the oracle."""
    M, N, K = 1023, 1025, 1027
    plan = g.sgemm_f32_plan_describe(M, N, K)
    print(f"[strip] plan {plan}", flush=True)
    # the tiles of the last tile column (one per tile row) compute the strip
    assert plan["strip_cols"] == 1 and plan["strip_tiles"] == plan["tiles"][0]
    A, B = wl.operands("c3", kind)
    _, dA, lda = device_matrix(A, K + 1)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N, N + 3)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    _check(A, B, c.result(), kind, ("c3", kind))


def test_strip_deterministic(gpu):
    M, N, K = 1023, 1025, 1027
    A, B = wl.operands("c3", "float")
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    first = None
    for i in range(10):
        c = GuardedC(M, N)
        run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
        gpu.cuda.synchronize()
        r = c.result().view(np.uint32).copy()
        if first is None:
            first = r
        else:
            assert np.array_equal(r, first), f"run {i} differs from run 0"
