"""Stream-K through the C ABI: the last tiles' K-panel units are shared out over the
resident workgroups, partial tiles go through a caller workspace, and a fixup kernel adds
them in ascending K order. Checked against the oracle (exact on small integers), with
guard bands around C and NaN in the workspace and the operands' row padding, for the
automatic plan and for every tile variant forced into stream-K on shapes that reach each
form of the partition: every tile shared, plain tiles followed by shared ones, fewer
units than workgroups, and ranges that start with a whole tile."""
import math

import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl
from gpu_util import TOL, GuardedC, device_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return torch


def streamk_variants():
    return g.streamk_variants()


def shared_c3_variant():
    """A variant whose stream-K form shares every tile of the ragged 1023x1025x1027 shape
    (64 x 64 tiles, two workgroups per CU: 272 tiles, fewer than the 512 workgroups)."""
    return g.variant_names().index("mfma_64x64x32_w2x1_kg2_dl")


def run_streamk(torch, A, B, variant=-1, ldc=None, lda=None, ldb=None, ws_fill=float("nan")):
    M, K = A.shape
    N = B.shape[1]
    _, dA, lda = device_matrix(A, lda)
    _, dB, ldb = device_matrix(B, ldb)
    c = GuardedC(M, N, ldc)
    ws_bytes = g.sgemm_f32_streamk_workspace_size(M, N, K, lda, ldb, c.ldc, variant=variant)
    ws = torch.full((max(ws_bytes // 4, 1) + 64,), ws_fill, device="cuda")
    d = g.sgemm_f32_streamk_describe(M, N, K, variant)
    print(f"[streamk] {M}x{N}x{K} variant {variant} plan {d}", flush=True)
    assert d["partition_ok"]
    g.sgemm_f32_streamk(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, c.ptr, c.ldc, variant,
                        ws.data_ptr(), ws_bytes)
    torch.cuda.synchronize()
    return c.result(), d


def hybrid_shape(variant):
    """A square-ish shape whose tile count is at least 2 G + G/8 for this variant: a round
    of plain tiles, then the shared ones; M, N and K are ragged."""
    d0 = g.sgemm_f32_streamk_describe(64, 64, 64, variant)
    BM, BN, BK = d0["BM"], d0["BN"], d0["BK"]
    G = g.sgemm_f32_streamk_describe(BM, BN, BK * 4096, variant)["G"]   # G at full size
    side = math.ceil(math.sqrt(2 * G + G // 8))
    return side * BM - 3, side * BN - 5, 3 * BK + 5


# every variant with a stream-K form (the table is read on the host, no GPU needed)
VARIANT_SLOTS = g.streamk_variants()


@pytest.mark.parametrize("variant", [-1] + VARIANT_SLOTS)
@pytest.mark.parametrize("M,N,K", [(1023, 1025, 1027), (300, 257, 129), (65, 65, 33),
                                   (1, 1, 300), (130, 70, 1000)])
def test_streamk_exact_integers(gpu, variant, M, N, K):
    if variant >= 0 and variant not in streamk_variants():
        pytest.skip("variant has no stream-K form")
    rng = np.random.default_rng(M + 7 * N + 13 * K + variant)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    C, d = run_streamk(gpu, A, B, variant, ldc=N + 3, lda=K + 1, ldb=N + 2)
    if variant >= 0:
        assert d["streamk"] or d["tiles"] % d["G"] == 0
    rep = oracle.check(A, B, C)
    assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, rep


@pytest.mark.parametrize("variant", VARIANT_SLOTS)
def test_streamk_plain_then_shared_tiles(gpu, variant):
    if variant not in streamk_variants():
        pytest.skip("variant has no stream-K form")
    M, N, K = hybrid_shape(variant)
    rng = np.random.default_rng(variant + 101)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    C, d = run_streamk(gpu, A, B, variant)
    assert d["streamk"] and d["tiles_dp"] > 0, d
    rep = oracle.check(A, B, C)
    assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, rep


@pytest.mark.parametrize("name", ["c3", "c2", "c1", "sk"])
def test_streamk_workloads_float(gpu, name):
    A, B = wl.operands(name)
    C, d = run_streamk(gpu, A, B)
    if name == "sk":
        assert d["streamk"]
    rep = oracle.check(A, B, C)
    assert rep["max_err"] <= TOL and rep["n_nonfinite"] == 0, rep


def test_streamk_large_ragged_sampled(gpu):
    """The ragged 4500x4500x8192 workload with the register-panel kernel's stream-K form
    forced: every 256 x 256 tile shared out as stream-K units (18 x 18 tiles on 256
    workgroups). Sampled rows, each over every column, against the oracle: first and last
    rows of tile rows and the ragged last tile row."""
    A, B = wl.operands("rk")
    rp = g.variant_names().index("mfma_256x256x32_w2x2_rp")
    C, d = run_streamk(gpu, A, B, rp)
    assert d["streamk"] and d["name"] == "mfma_256x256x32_w2x2_rp", d
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 255, 256, 2047, 4095, 4096, 4351, 4352, 4480, 4498, 4499,
                   *rng.integers(0, 4500, 20).tolist()})
    rep = oracle.check(A, B, C, rows=rows)
    assert rep["max_err"] <= TOL and rep["n_nonfinite"] == 0, rep
    assert rep["n_checked"] == len(rows) * 4500


def test_streamk_deterministic(gpu):
    A, B = wl.operands("c3")
    v = shared_c3_variant()
    first, d = run_streamk(gpu, A, B, v)
    first = first.copy()
    assert d["streamk"] and d["shared_tiles"] > 0
    rep = oracle.check(A, B, first)
    assert rep["max_err"] <= TOL and rep["n_nonfinite"] == 0, rep
    for fill in (0.0, 1e30, float("nan")):
        again, _ = run_streamk(gpu, A, B, v, ws_fill=fill)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_streamk_plain_plan_matches_hot_path(gpu):
    """Where the plan keeps the plain grid, the result is sgemm_f32's, bit for bit."""
    torch = gpu
    A, B = wl.operands("c2")
    C, d = run_streamk(torch, A, B)
    assert not d["streamk"]
    ref = g.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(C.view(np.uint32), ref.cpu().numpy().view(np.uint32))


def test_streamk_edges(gpu):
    torch = gpu
    lib = g.library()
    _, dA, _ = device_matrix(np.ones((40, 1), np.float32))
    _, dB, _ = device_matrix(np.ones((1, 30), np.float32))
    c = GuardedC(40, 30)
    ws = torch.zeros(1024, device="cuda")
    # K = 0: C is the empty sum
    g.sgemm_f32_streamk(40, 30, 0, dA.data_ptr(), 1, dB.data_ptr(), 30, c.ptr, c.ldc, -1,
                        ws.data_ptr(), 4096)
    torch.cuda.synchronize()
    assert (c.result() == 0).all()
    # a workspace smaller than the plan needs is refused before anything runs
    M, N, K = 1023, 1025, 1027
    v = shared_c3_variant()
    need = g.sgemm_f32_streamk_workspace_size(M, N, K, variant=v)
    assert need > 0
    big = torch.zeros(need // 4 + 64, device="cuda")
    _, dA, _ = device_matrix(np.ones((M, K), np.float32))
    _, dB, _ = device_matrix(np.ones((K, N), np.float32))
    c = GuardedC(M, N)
    rc = lib.sgemm_f32_streamk(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, c.ptr, N, v,
                               big.data_ptr(), need - 4, None)
    assert rc == -6
    torch.cuda.synchronize()
    assert np.isnan(c.result()).all()    # nothing was written
