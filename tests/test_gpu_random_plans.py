"""The automatic plan (sgemm_f32) on shapes drawn from a fixed seed: ragged and square, one
tile per CU and many, short and deep K, with padded leading dimensions (NaN in A's and B's
padding, guard cells around C). Whatever the plan takes for each (tile variant, column strip
in either form, the persistent kernel with its edge launches), small-integer inputs make the
check against the oracle exact."""
import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl
from gpu_util import GuardedC, device_matrix, run_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return torch


def drawn_shapes(n=40, seed=2026, max_macs=2.5e9):
    """Log-uniform M, N, K in [1, 3000], at most max_macs multiply-adds each, and padding
    of 0-9 extra floats per row (C's padding a multiple of 8 half of the time)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M, N, K = (int(round(np.exp(rng.uniform(0.0, np.log(3000.0))))) for _ in range(3))
        if M * N * K > max_macs:
            continue
        pa, pb = int(rng.integers(0, 10)), int(rng.integers(0, 10))
        pc = int(rng.integers(0, 2)) * 8 if rng.integers(0, 2) else int(rng.integers(0, 10))
        out.append((M, N, K, K + pa, N + pb, N + pc))
    return out


# shapes that reach the column strip's two forms and the persistent kernel's edges
DESIGNED = [(1023, 1025, 1027, 1030, 1025, 1032), (2047, 2049, 700, 700, 2053, 2049),
            (8192, 8193, 256, 257, 8193, 8200), (6144, 6145, 512, 515, 6145, 6145),
            (8200, 8200, 128, 128, 8200, 8200), (4173, 4096, 96, 97, 4100, 4104)]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", drawn_shapes() + DESIGNED)
def test_auto_plan_exact(gpu, M, N, K, lda, ldb, ldc):
    plan = g.sgemm_f32_plan_describe(M, N, K, lda=lda, ldb=ldb, ldc=ldc)
    rng = np.random.default_rng(M * 7 + N * 13 + K * 17)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, _ = device_matrix(A, lda)
    _, dB, _ = device_matrix(B, ldb)
    c = GuardedC(M, N, ldc)
    print(f"[random] {M}x{N}x{K} lda={lda} ldb={ldb} ldc={ldc} -> {plan['name']} "
          f"strip {plan['strip_cols']}/{plan['strip_rows']} edges {plan['edge_launches']}",
          flush=True)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    rows = None
    if M > 2048:
        # every row of the last 300 (bottom edges, last tile rows) and a spread of others
        rows = sorted(set(range(M - 300, M)) | set(range(0, M, 97)))
    rep = oracle.check(A, B, c.result(), rows=rows)
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, (M, N, K, plan["name"], rep)
