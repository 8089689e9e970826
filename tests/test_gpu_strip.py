"""The column strip through the C ABI: when N leaves one to four columns past the last whole
tile column, the tiles also compute those columns, on the vector ALUs between their MFMAs:
spread over the tiles of each row (each tile a few of the row's strip rows, from its A
panels in LDS; up to the variant's strip_cols_max columns), or, for one column when the
tile columns are too few for that, by the last tile column from the A operands it reads for
the MFMAs. Checked against the oracle (exact on small integers, within the normalised
tolerance on floats) with NaN-poisoned row padding and guard bands around C, for every
strip-capable variant forced (both forms, every strip width), for the automatic plan, and
for run-to-run determinism."""
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
    """(M, N, K) with N = (whole tile columns) + 1 (or + 2), K on both sides of the panel
    depth and of K-group rounds (with partial last panels), M ragged: products of a few
    tiles, where a strip would save no round of tiles, so the plan masks a last tile
    column that holds one or two valid columns instead (the strip forms are covered by
    test_strip_forced_both_forms)."""
    bn = g.sgemm_f32_variant_info(v)["BN"]
    return [(63, 5 * bn + 1, 33), (130, 8 * bn + 1, 256), (200, 5 * bn + 1, 257),
            (65, 17 * bn + 1, 300), (257, 5 * bn + 1, 5), (129, 6 * bn + 1, 1),
            (70, 5 * bn + 1, 2050), (17, 9 * bn + 1, 4353), (100, 5 * bn + 1, 37),
            (33, 7 * bn + 1, 64), (65, bn + 1, 300), (130, 2 * bn + 1, 129),
            (130, 5 * bn + 2, 256)]


def forced_strip_shapes(v, cus):
    """Shapes on which variant v, forced, computes a column strip, for a device of `cus`
    compute units: one tile per CU with a one-column remainder, whose masked 17th (or
    second) tile column would take a second round. Sixteen tile columns spread the strip's
    rows four or eight to a tile, seventeen leave the last tile column without rows, and
    one tile column leaves them all to it (the last-column form)."""
    info = g.sgemm_f32_variant_info(v)
    bm, bn = info["BM"], info["BN"]
    return [((cus // 16) * bm - 3, 16 * bn + 1, 33, "spread"),
            ((cus // 17) * bm, 17 * bn + 1, 72, "spread"),
            (cus * bm - 5, bn + 1, 40, "column")]


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


def test_masked_last_column_forced(gpu):
    for v in strip_variants():
        _strip_shapes(gpu, v)


def _strip_shapes(gpu, v):
    name = g.variant_names()[v]
    for (M, N, K) in shapes_for(v):
        rng = np.random.default_rng(M * 7919 + N * 31 + K)
        A = wl.draw(rng, (M, K), "int")
        B = wl.draw(rng, (K, N), "int")
        for lda, ldb, ldc in [(K + 3, N + 5, N + 2), (K, N, N)]:
            d = g.sgemm_f32_variant_describe(v, M, N, K, lda, ldb, ldc)
            assert d["strip_cols"] == 0 and d["tiles"][1] * d["BN"] >= N, (name, d)
            _, dA, _ = device_matrix(A, lda)
            _, dB, _ = device_matrix(B, ldb)
            c = GuardedC(M, N, ldc)
            print(f"[strip] {name} {M}x{N}x{K} lda={lda} ldb={ldb} ldc={ldc}", flush=True)
            run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
            gpu.cuda.synchronize()
            _check(A, B, c.result(), "int", (name, M, N, K, lda, ldb, ldc))


def test_strip_forced_both_forms(gpu):
    """Every strip-capable variant forced where its plan computes the strip: spread over
    the tile rows and in the last tile column, as variant_describe reports; exact on
    integers with padded leading dimensions and guard bands."""
    cus = gpu.cuda.get_device_properties(0).multi_processor_count
    for v in strip_variants():
        name = g.variant_names()[v]
        for (M, N, K, form) in forced_strip_shapes(v, cus):
            lda, ldb, ldc = K + 1, N + 3, N + 2
            d = g.sgemm_f32_variant_describe(v, M, N, K, lda, ldb, ldc)
            assert d["variant"] == v and d["strip_cols"] == 1, (name, M, N, K, d)
            assert (d["strip_rows"] > 0) == (form == "spread"), (name, M, N, K, d)
            rng = np.random.default_rng(M + 3 * N + 7 * K)
            A = wl.draw(rng, (M, K), "int")
            B = wl.draw(rng, (K, N), "int")
            _, dA, _ = device_matrix(A, lda)
            _, dB, _ = device_matrix(B, ldb)
            c = GuardedC(M, N, ldc)
            print(f"[strip] {name} {M}x{N}x{K} {form} rows={d['strip_rows']}", flush=True)
            run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
            gpu.cuda.synchronize()
            _check(A, B, c.result(), "int", (name, M, N, K, form))


def test_strip_forced_wide(gpu):
    """Every strip-capable variant forced on shapes whose N leaves two, three or four
    columns (up to the variant's strip_cols_max): the spread form takes them all, as
    variant_describe reports; exact on integers with padded leading dimensions and guard
    bands, K below, at and past the panel depth."""
    cus = gpu.cuda.get_device_properties(0).multi_processor_count
    for v in strip_variants():
        info = g.sgemm_f32_variant_info(v)
        name, bm, bn = info["name"], info["BM"], info["BN"]
        for sc in range(2, info["strip_cols_max"] + 1):
            for (M, N, K) in [((cus // 16) * bm - 3, 16 * bn + sc, 33),
                              ((cus // 17) * bm, 17 * bn + sc, 72 + sc)]:
                lda, ldb, ldc = K + 1, N + 3, N + 2
                d = g.sgemm_f32_variant_describe(v, M, N, K, lda, ldb, ldc)
                assert d["strip_cols"] == sc and d["strip_rows"] > 0, (name, M, N, K, d)
                rng = np.random.default_rng(M + 3 * N + 7 * K + sc)
                A = wl.draw(rng, (M, K), "int")
                B = wl.draw(rng, (K, N), "int")
                _, dA, _ = device_matrix(A, lda)
                _, dB, _ = device_matrix(B, ldb)
                c = GuardedC(M, N, ldc)
                print(f"[strip] {name} {M}x{N}x{K} {sc} columns rows={d['strip_rows']}",
                      flush=True)
                run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
                gpu.cuda.synchronize()
                _check(A, B, c.result(), "int", (name, M, N, K, sc))


def test_row_strip_forced(gpu):
    """Every strip-capable variant forced on shapes whose M leaves one to strip_cols_max
    rows past the last whole tile row: the tiles of each tile column compute those rows
    (each tile row a share of the columns), as variant_describe reports; exact on
    integers with padded leading dimensions, guard bands and a ragged, masked last tile
    column."""
    cus = gpu.cuda.get_device_properties(0).multi_processor_count
    for v in strip_variants():
        info = g.sgemm_f32_variant_info(v)
        name, bm, bn = info["name"], info["BM"], info["BN"]
        for rr in range(1, info["strip_cols_max"] + 1):
            for (M, N, K) in [(16 * bm + rr, (cus // 16) * bn - 3, 33),
                              (17 * bm + rr, (cus // 17) * bn, 72 + rr)]:
                lda, ldb, ldc = K + 3, N + 1, N + 2
                d = g.sgemm_f32_variant_describe(v, M, N, K, lda, ldb, ldc)
                assert d["row_strip"] == rr and d["strip_cols"] == 0, (name, M, N, K, d)
                assert d["tiles"][0] == M // bm, d
                rng = np.random.default_rng(7 * M + N + 3 * K)
                A = wl.draw(rng, (M, K), "int")
                B = wl.draw(rng, (K, N), "int")
                _, dA, _ = device_matrix(A, lda)
                _, dB, _ = device_matrix(B, ldb)
                c = GuardedC(M, N, ldc)
                print(f"[strip] {name} {M}x{N}x{K} {rr} strip rows, "
                      f"{d['row_strip_cols']} columns per tile", flush=True)
                run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
                gpu.cuda.synchronize()
                _check(A, B, c.result(), "int", (name, M, N, K, rr))


@pytest.mark.parametrize("M,N,K", [(1025, 1024, 1024), (1028, 1024, 1027), (2049, 2048, 2048),
                                   (513, 512, 4096), (1026, 11934, 230)])
def test_plan_row_strip(gpu, M, N, K):
    """The automatic plan where M leaves one to four rows past the tile rows: a row strip,
    matching the oracle (floats, normalised tolerance; sampled rows, the strip's included,
    at the larger sizes)."""
    plan = g.sgemm_f32_plan_describe(M, N, K)
    print(f"[strip] plan {M}x{N}x{K} {plan}", flush=True)
    assert plan["row_strip"] == M % plan["BM"] and plan["row_strip_cols"] > 0, plan
    rng = np.random.default_rng(M * 13 + N * 5 + K)
    A = wl.draw(rng, (M, K), "uniform")
    B = wl.draw(rng, (K, N), "uniform")
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N, N + 1)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    C = c.result()
    if M * N * K <= 2 ** 31:
        rep = oracle.check(A, B, C)
    else:
        rep = oracle.check(A, B, C, rows=np.unique(np.r_[0:4, 1000:1004, M - 12:M]))
    assert rep["n_nonfinite"] == 0 and rep["max_err"] <= TOL, rep


@pytest.mark.parametrize("M,N,K", [(1024, 1026, 1024), (1024, 1027, 1024), (1023, 1028, 1027),
                                   (2048, 2050, 2048), (512, 514, 4096)])
def test_plan_wide_strip(gpu, M, N, K):
    """The automatic plan where N leaves two to four columns past the tile columns: it puts
    them in a spread strip, and the result matches the oracle (floats, normalised
    tolerance; sampled rows at the larger size)."""
    plan = g.sgemm_f32_plan_describe(M, N, K)
    print(f"[strip] plan {M}x{N}x{K} {plan}", flush=True)
    assert plan["strip_cols"] == N % plan["BN"] and plan["strip_rows"] > 0, plan
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    A = wl.draw(rng, (M, K), "uniform")
    B = wl.draw(rng, (K, N), "uniform")
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N, N + 1)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    C = c.result()
    rows = None if M * N * K <= 2 ** 31 else np.unique(np.r_[0:8, M - 8:M, 1000:1010])
    rep = oracle.check(A, B, C, rows=rows) if rows is not None else oracle.check(A, B, C)
    assert rep["n_nonfinite"] == 0 and rep["max_err"] <= TOL, rep


@pytest.mark.parametrize("kind", ["int", "float"])
def test_ragged_workload_plan_uses_strip(gpu, kind):
    """The ragged 1023 x 1025 x 1027 workload: the plan puts its last column in a strip, and
    the result matches the oracle."""
    M, N, K = 1023, 1025, 1027
    plan = g.sgemm_f32_plan_describe(M, N, K)
    print(f"[strip] plan {plan}", flush=True)
    # every tile computes four of its row's 64 strip rows
    assert plan["strip_cols"] == 1 and plan["strip_rows"] == 4
    assert plan["strip_tiles"] == plan["tiles"][0] * plan["tiles"][1]
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
