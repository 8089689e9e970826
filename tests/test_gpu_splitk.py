"""Split-K through the C ABI: the (tile, K-range) items of the hot kernel write partial
products into a caller workspace and a second kernel sums them in fixed order. Checked
against the oracle (exact on small integers), with guard bands around C, for explicit
and automatic split counts, ragged K, and bit-identical repeats."""
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


def run_splitk(torch, A, B, splits, ldc=None, lda=None, ldb=None):
    M, K = A.shape
    N = B.shape[1]
    _, dA, lda = device_matrix(A, lda)
    _, dB, ldb = device_matrix(B, ldb)
    c = GuardedC(M, N, ldc)
    ws_bytes = g.sgemm_f32_splitk_workspace_size(M, N, K, splits)
    ws = torch.full((max(ws_bytes // 4, 1) + 64,), float("nan"), device="cuda")
    print(f"[splitk] {M}x{N}x{K} splits {splits} ws {ws_bytes}", flush=True)
    g.sgemm_f32_splitk(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, c.ptr, c.ldc, splits,
                       ws.data_ptr(), ws_bytes)
    torch.cuda.synchronize()
    return c.result()


@pytest.mark.parametrize("M,N,K,splits", [
    (256, 256, 8192, 2), (256, 256, 8192, 3), (256, 256, 8192, 8), (256, 256, 8192, 0),
    (64, 48, 4096, 4), (130, 70, 1000, 5), (1, 1, 300, 3), (1023, 1025, 1027, 2),
    (1023, 1025, 1027, 3), (300, 200, 65, 32), (517, 259, 2049, 0)])
def test_splitk_exact_integers(gpu, M, N, K, splits):
    rng = np.random.default_rng(M + 7 * N + 13 * K + splits)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    C = run_splitk(gpu, A, B, splits, ldc=N + 3, lda=K + 1, ldb=N + 2)
    rep = oracle.check(A, B, C)
    assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, rep


@pytest.mark.parametrize("name,splits", [("c2", 4), ("c3", 2), ("c3", 0), ("sk", 0), ("sk", 32)])
def test_splitk_configs_float(gpu, name, splits):
    A, B = wl.operands(name)
    C = run_splitk(gpu, A, B, splits)
    rep = oracle.check(A, B, C)
    assert rep["max_err"] <= TOL and rep["n_nonfinite"] == 0, rep


def test_splitk_deterministic(gpu):
    rng = np.random.default_rng(3)
    A = wl.draw(rng, (256, 8192), "uniform")
    B = wl.draw(rng, (8192, 256), "uniform")
    first = run_splitk(gpu, A, B, 4).copy()
    rep = oracle.check(A, B, first)
    assert rep["max_err"] <= TOL, rep
    for _ in range(5):
        again = run_splitk(gpu, A, B, 4)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
