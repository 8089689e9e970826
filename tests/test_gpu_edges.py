"""Edge cases of every kernel through the C ABI: ragged sizes around the tile sizes,
NaN-poisoned row padding of A and B (lda > K, ldb > N), guard bands around C
(ldc > N, a row above and below), misaligned base pointers, K == 0, M == 0,
determinism and a non-default stream. Small-integer inputs make every check exact."""
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


SIZES = [1, 2, 3, 5, 31, 32, 33, 47, 48, 49, 63, 64, 65, 79, 80, 81, 127, 128, 129, 255, 257]
SHAPES = sorted({(s, 65, 33) for s in SIZES} | {(65, s, 33) for s in SIZES} |
                {(65, 33, s) for s in SIZES} |
                {(257, 255, 129), (129, 257, 255), (300, 520, 9), (7, 600, 600),
                 (600, 7, 600), (513, 511, 68), (260, 260, 260),
                 # K % 4 == 0 but not a multiple of the panel depth
                 (65, 33, 4), (65, 33, 36), (33, 300, 100), (270, 130, 20)})


def kernels_for():
    return ["auto", "naive", "tiled16", "tiled32"] + [f"v{v}" for v in range(len(g.variant_names()))]


def exact_check(A, B, C, what):
    rep = oracle.check(A, B, C)
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, (what, rep)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_ragged_shapes_padded_and_guarded(gpu, M, N, K):
    rng = np.random.default_rng(M * 1000003 + N * 1009 + K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    # padded rows (NaN in the padding, odd leading dimensions) and a padded, guarded C
    for lda, ldb, ldc in [(K + 3, N + 5, N + 2), (K, N, N)]:
        _, dA, _ = device_matrix(A, lda)
        _, dB, _ = device_matrix(B, ldb)
        for kern in kernels_for():
            c = GuardedC(M, N, ldc)
            print(f"[edge] {M}x{N}x{K} lda={lda} ldb={ldb} ldc={ldc} {kern}", flush=True)
            run_kernel(kern, M, N, K, dA, lda, dB, ldb, c)
            gpu.cuda.synchronize()
            exact_check(A, B, c.result(), (M, N, K, lda, ldb, ldc, kern))


@pytest.mark.parametrize("M,N,K", [(257, 129, 65), (64, 64, 64), (1, 1, 1), (300, 301, 302),
                                   (300, 260, 132)])
def test_misaligned_pointers(gpu, M, N, K):
    """Bases one or three floats past 16-byte alignment: every kernel still works (the hot
    kernel's 16-byte buffer loads and stores only need 4-byte alignment)."""
    rng = np.random.default_rng(7)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A, offset=1)
    _, dB, ldb = device_matrix(B, offset=3)
    for kern in kernels_for():
        c = GuardedC(M, N, offset=1)
        print(f"[edge] misaligned {M}x{N}x{K} {kern}", flush=True)
        run_kernel(kern, M, N, K, dA, lda, dB, ldb, c)
        gpu.cuda.synchronize()
        exact_check(A, B, c.result(), ("misaligned", kern))


@pytest.mark.parametrize("kern", ["auto", "naive", "tiled16", "tiled32", "v0"])
def test_k_zero_and_empty(gpu, kern):
    dummy = gpu.zeros(16, device="cuda")
    c = GuardedC(70, 90, 93)
    run_kernel(kern, 70, 90, 0, dummy, 1, dummy, 90, c)
    gpu.cuda.synchronize()
    assert (c.result() == 0).all()
    c0 = GuardedC(0, 90)
    run_kernel(kern, 0, 90, 5, dummy, 5, dummy, 90, c0)
    gpu.cuda.synchronize()
    c0.result()


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_deterministic(gpu, name):
    """Twenty back-to-back runs give identical bits (no atomics, no races)."""
    w = wl.WORKLOADS[name]
    A, B = wl.operands(name)
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    out = gpu.empty((w.M, w.N), device="cuda")
    first = None
    for i in range(20):
        g.sgemm_f32(w.M, w.N, w.K, dA.data_ptr(), lda, dB.data_ptr(), ldb, out.data_ptr(), w.N)
        gpu.cuda.synchronize()
        got = out.cpu().numpy().copy()
        if first is None:
            first = got
            rep = oracle.check(A, B, got)
            assert rep["max_err"] <= TOL and rep["n_nonfinite"] == 0, rep
        else:
            assert np.array_equal(first.view(np.uint32), got.view(np.uint32)), f"run {i} differs"


def test_side_stream_and_matmul(gpu):
    """The tensor layer launches on torch's current stream; a side stream works."""
    A, B = wl.operands("c3")
    dA = gpu.from_numpy(A).cuda()
    dB = gpu.from_numpy(B).cuda()
    s = gpu.cuda.Stream()
    with gpu.cuda.stream(s):
        C = g.matmul(dA, dB)
    s.synchronize()
    rep = oracle.check(A, B, C.cpu().numpy())
    assert rep["max_err"] <= TOL, rep
    Cn = g.matmul(dA, dB, kernel="naive")
    gpu.cuda.synchronize()
    assert oracle.check(A, B, Cn.cpu().numpy())["max_err"] <= TOL
