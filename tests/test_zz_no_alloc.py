"""The no-allocation stream-K entry point (sgemm_f32_streamk_noalloc) through the C ABI:
its partial tiles go to the library's static per-GPU scratch instead of a caller
workspace. Its results must equal sgemm_f32_streamk's with a workspace bit for bit (same
plan, same kernels, same summation order) and pass the oracle: exact on small integers,
within the normalised tolerance on floats. Calls follow each other on one stream, the
second on a smaller input than the first, so the second reuses scratch the first left
behind."""
import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl
from gpu_util import TOL, GuardedC, device_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return t


def _operands(M, N, K, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "int":
        return wl.draw(rng, (M, K), "int"), wl.draw(rng, (K, N), "int")
    return wl.draw(rng, (M, K), "uniform"), wl.draw(rng, (K, N), "uniform")


def _noalloc(torch, A, B, variant):
    M, K = A.shape
    N = B.shape[1]
    _, dA, lda = device_matrix(A, K + 3)           # NaN row padding must not leak
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N)
    rc = g.library().sgemm_f32_streamk_noalloc(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                                               c.ptr, c.ldc, variant, None)
    torch.cuda.synchronize()
    return rc, c.result()


def _with_workspace(torch, A, B, variant):
    M, K = A.shape
    N = B.shape[1]
    _, dA, lda = device_matrix(A, K + 3)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N)
    ws_bytes = g.sgemm_f32_streamk_workspace_size(M, N, K, lda, ldb, c.ldc, variant=variant)
    ws = torch.full((max(ws_bytes // 4, 1),), float("nan"), device="cuda")
    g.sgemm_f32_streamk(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, c.ptr, c.ldc, variant,
                        ws.data_ptr(), ws_bytes)
    torch.cuda.synchronize()
    return c.result()


def _check(A, B, C, kind):
    rep = oracle.check(A, B, C)
    assert rep["n_nonfinite"] == 0, rep
    if kind == "int":
        assert rep["n_inexact"] == 0, rep
    else:
        assert rep["max_err"] <= TOL, rep


# (M, N, K, forced variant name or None): the first call is the larger one; each plan
# shares tiles, so its partial sums go through the scratch
CALLS = [(512, 512, 8192, None), (300, 200, 5000, None),
         (1023, 1025, 1027, "mfma_64x64x32_w2x1_kg2_dl")]


@pytest.mark.parametrize("kind", ["int", "float"])
def test_noalloc_matches_workspace_entry(torch, kind):
    names = g.variant_names()
    for i, (M, N, K, vname) in enumerate(CALLS):
        v = -1 if vname is None else names.index(vname)
        d = g.sgemm_f32_streamk_describe(M, N, K, v)
        print(f"[noalloc] {M}x{N}x{K} {kind} variant {v} plan {d['name']} "
              f"workspace {d['workspace_bytes']}", flush=True)
        assert d["streamk"] and 0 < d["workspace_bytes"] <= g.sgemm_f32_streamk_noalloc_scratch_bytes()
        A, B = _operands(M, N, K, kind, 500 + i)
        rc, C = _noalloc(torch, A, B, v)
        assert rc == 0, g.library().sgemm_f32_status_string(rc)
        ref = _with_workspace(torch, A, B, v)
        assert np.array_equal(C.view(np.uint32), ref.view(np.uint32)), \
            f"noalloc differs from the workspace entry at {M}x{N}x{K}"
        _check(A, B, C, kind)


def test_noalloc_plain_plan_and_scratch_limit(torch):
    # a plan that shares no tile runs the plain grid and needs no scratch
    M, N, K = 1023, 1025, 1027
    d = g.sgemm_f32_streamk_describe(M, N, K, -1)
    print(f"[noalloc] {M}x{N}x{K} auto plan {d['name']} streamk {d['streamk']}", flush=True)
    A, B = _operands(M, N, K, "int", 520)
    rc, C = _noalloc(torch, A, B, -1)
    assert rc == 0
    _check(A, B, C, "int")
    # a forced plan whose partial tiles exceed the scratch is refused before any launch
    rp = g.variant_names().index("mfma_256x256x32_w2x2_rp")
    d = g.sgemm_f32_streamk_describe(M, N, K, rp)
    assert d["workspace_bytes"] > g.sgemm_f32_streamk_noalloc_scratch_bytes()
    print(f"[noalloc] {M}x{N}x{K} forced {d['name']} needs {d['workspace_bytes']}", flush=True)
    rc, C = _noalloc(torch, A, B, rp)
    assert rc == -8
    assert np.isnan(C).all()      # nothing was written
    # then a small call still works
    A, B = _operands(130, 70, 3000, "float", 521)
    v = g.variant_names().index("mfma_64x64x32_w2x1_kg2_dl")
    rc, C = _noalloc(torch, A, B, v)
    assert rc == 0
    _check(A, B, C, "float")
    assert np.array_equal(C.view(np.uint32), _with_workspace(torch, A, B, v).view(np.uint32))
