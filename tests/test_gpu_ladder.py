"""The rungs of the pages' ladder beside the hot kernel, through the C ABI: scalar
register tiling (1-D 4x1 strip, 2-D 4x4 and 8x8) against the oracle, and the LDS
transpose microbenchmark (tile 32/64, padded or not) against the oracle's transpose."""
import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl
from gpu_util import TOL, GuardedC, device_matrix, SENTINEL

pytestmark = pytest.mark.gpu

TILES = [(4, 1), (4, 4), (8, 8)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return torch


@pytest.mark.parametrize("variant", ["int", "float"])
@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_regtiled_configs(gpu, name, variant):
    w = wl.WORKLOADS[name]
    A, B = wl.operands(name, variant)
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    for tm, tn in TILES:
        c = GuardedC(w.M, w.N)
        print(f"[ladder] {name} {variant} regtiled {tm}x{tn}", flush=True)
        g.sgemm_f32_regtiled(w.M, w.N, w.K, dA.data_ptr(), lda, dB.data_ptr(), ldb, c.ptr, c.ldc,
                             tm=tm, tn=tn)
        gpu.cuda.synchronize()
        rep = oracle.check(A, B, c.result())
        assert rep["n_nonfinite"] == 0, (tm, tn, rep)
        if variant == "int":
            assert rep["n_inexact"] == 0, (tm, tn, rep)
        else:
            assert rep["max_err"] <= TOL, (tm, tn, rep)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (65, 33, 9), (129, 127, 17), (7, 300, 64),
                                   (300, 7, 130), (257, 129, 31)])
def test_regtiled_ragged_padded(gpu, M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A, K + 3)
    _, dB, ldb = device_matrix(B, N + 1)
    for tm, tn in TILES:
        c = GuardedC(M, N, N + 3)
        print(f"[ladder] {M}x{N}x{K} regtiled {tm}x{tn}", flush=True)
        g.sgemm_f32_regtiled(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, c.ptr, c.ldc,
                             tm=tm, tn=tn)
        gpu.cuda.synchronize()
        rep = oracle.check(A, B, c.result())
        assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, (tm, tn, rep)


@pytest.mark.parametrize("rows,cols", [(1, 1), (32, 32), (64, 64), (33, 95), (1000, 7),
                                       (257, 1023), (2048, 2048)])
def test_lds_transpose(gpu, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    X = rng.standard_normal((rows, cols)).astype(np.float32)
    expect = oracle.transpose(X)
    _, dX, ldi = device_matrix(X, cols + 2)
    for tile in (32, 64):
        for pad in (0, 1):
            ldo = rows + 3
            out = gpu.full(((cols + 1) * ldo,), float(SENTINEL), device="cuda")
            print(f"[ladder] transpose {rows}x{cols} tile {tile} pad {pad}", flush=True)
            g.sgemm_f32_lds_transpose(rows, cols, dX.data_ptr(), ldi, out.data_ptr(), ldo,
                                      tile=tile, pad=pad)
            gpu.cuda.synchronize()
            o = out.cpu().numpy()
            got = o[: cols * ldo].reshape(cols, ldo)
            assert np.array_equal(got[:, :rows], expect), (tile, pad)
            assert (got[:, rows:] == SENTINEL).all() and (o[cols * ldo:] == SENTINEL).all()
