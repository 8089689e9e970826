"""Parity of the HIP kernels with the CPU oracle, through the C ABI.

The five workloads run on every kernel of the library (the naive and scalar-tiled rungs
skip the 8192^3 shape, which only the hot path needs). Small-integer inputs must match
the oracle exactly (every partial sum is an integer below 2^24, so any summation order
is exact in FP32); float inputs must have max |C - C_ref| / sum_k |a_ik b_kj| <= 1e-5.
At the full sizes the oracle checks sampled rows (all their columns), chosen to cover
tile edges. Every call also checks that nothing outside C's M x N region was written.
"""
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
    g.library()   # raises if the HIP library is missing: no fallback
    return torch


def sample_rows(M: int, n_random: int, seed: int):
    """Rows at tile boundaries (multiples of 32/64/128/256 and their neighbours) plus
    random rows."""
    if M <= 2048:
        return None   # the oracle checks every row
    edges = {0, 1, M - 1, M - 2}
    for t in (32, 64, 128, 256):
        for r in range(t, M, max(t, M // 8)):
            edges.update({r - 1, r})
    rng = np.random.default_rng(seed)
    rows = sorted(edges | set(rng.choice(M, n_random, replace=False).tolist()))
    return [r for r in rows if 0 <= r < M]


def run_config(name, variant, kernel, torch):
    w = wl.WORKLOADS[name]
    A, B = wl.operands(name, variant)
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(w.M, w.N)
    print(f"[parity] {name} {variant} {kernel} {w.M}x{w.N}x{w.K}", flush=True)
    run_kernel(kernel, w.M, w.N, w.K, dA, lda, dB, ldb, c)
    torch.cuda.synchronize()
    C = c.result()
    rows = sample_rows(w.M, 24, seed=w.index)
    rep = oracle.check(A, B, C, rows=rows)
    assert rep["n_nonfinite"] == 0, rep
    if variant == "int":
        assert rep["n_inexact"] == 0, rep
    else:
        assert rep["max_err"] <= TOL, rep
    return rep


@pytest.mark.parametrize("variant", ["int", "float"])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_hot_path_configs(gpu, name, variant):
    run_config(name, variant, "auto", gpu)


@pytest.mark.parametrize("kernel", ["naive", "tiled16", "tiled32", "tiled32p"])
@pytest.mark.parametrize("variant", ["int", "float"])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_reference_kernels_configs(gpu, name, variant, kernel):
    run_config(name, variant, kernel, gpu)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_every_variant_on_configs(gpu, name):
    """Each tile variant of the hot kernel, forced, on the 1024-class shapes."""
    w = wl.WORKLOADS[name]
    A, B = wl.operands(name, "int")
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    for v, vname in enumerate(g.variant_names()):
        c = GuardedC(w.M, w.N)
        print(f"[parity] {name} int variant {vname}", flush=True)
        run_kernel(f"v{v}", w.M, w.N, w.K, dA, lda, dB, ldb, c)
        gpu.cuda.synchronize()
        rep = oracle.check(A, B, c.result())
        assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, (vname, rep)


AT_SCALE = [(2048, 2048, 2048), (3000, 3000, 3000), (16384, 16384, 256), (4096, 4096, 4096),
            (1200, 1200, 500), (1279, 1279, 2000), (1100, 1100, 1100),
            (1100, 1100, 4096), (512, 512, 4096), (1024, 512, 2048), (383, 385, 16387),
            (1516, 8811, 39)]


@pytest.mark.parametrize("M,N,K", AT_SCALE)
def test_planned_variants_at_scale(gpu, M, N, K):
    """Every tile variant the plan picks, at a size where it picks it (the mid-size shapes
    of the plan's fit), on small-integer inputs: exact on sampled rows at tile edges."""
    plan = g.sgemm_f32_plan_describe(M, N, K)
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A)
    _, dB, ldb = device_matrix(B)
    c = GuardedC(M, N)
    print(f"[parity] {M}x{N}x{K} int auto -> {plan['name']}", flush=True)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    rep = oracle.check(A, B, c.result(), rows=sample_rows(M, 16, seed=M))
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, (plan["name"], rep)


# The one-wave-per-SIMD variant forced onto ragged large shapes with NaN-padded leading
# dimensions: a partial last K-panel (K % 32 != 0, and K % 4 != 0), tiles that hold A's last
# rows and B's last columns, and a shape with fewer than one panel. The automatic plan only
# sends it shapes of many whole tiles, so these cases are forced.
RP_FORCED = [(4095, 4097, 4103), (2300, 1800, 3001), (3000, 2600, 20)]


@pytest.mark.parametrize("M,N,K", RP_FORCED)
def test_regpanel_variant_forced_ragged(gpu, M, N, K):
    v = g.variant_names().index("mfma_256x256x32_w2x2_rp")
    rng = np.random.default_rng(M + 5 * N + 11 * K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A, K + 3)
    _, dB, ldb = device_matrix(B, N + 5)
    c = GuardedC(M, N, N + 2)
    print(f"[parity] {M}x{N}x{K} int forced v{v} lda={lda} ldb={ldb}", flush=True)
    run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    rep = oracle.check(A, B, c.result(), rows=sample_rows(M, 16, seed=N))
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, rep


# The persistent variant (one workgroup per CU walking 128 x 256 tiles, each tile's C stored
# among the next tile's MFMAs) forced onto: the low-K workload; a ragged shape (whole-tile
# part on the kernel, right and bottom strips on the plan, K % 32 != 0); K with a partial
# second panel (33), three panels (96, the per-tile panel loop), four with a partial last
# (100); fewer tiles than CUs; tile counts that give workgroups an odd and an even number of
# tiles (the odd ones end on an empty tile); and a K of one panel, which goes to the plan.
# Leading dimensions are padded with NaN, so a read past a row's end shows in C.
PS_FORCED = [(16384, 16384, 64), (4095, 4097, 4103), (1024, 2048, 33), (2048, 1024, 96),
             (896, 1280, 100), (256, 512, 128), (128 * 25, 256 * 31, 64), (640, 768, 20)]


@pytest.mark.parametrize("name", ["mfma_128x256x32_w2x2_ps", "mfma_128x256x32_w2x4_ps"])
@pytest.mark.parametrize("M,N,K", PS_FORCED)
def test_persistent_variant_forced(gpu, M, N, K, name):
    v = g.variant_names().index(name)
    rng = np.random.default_rng(M + 7 * N + 13 * K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A, K + 3)
    _, dB, ldb = device_matrix(B, N + 5)
    c = GuardedC(M, N, N + 2)
    print(f"[parity] {M}x{N}x{K} int forced v{v} lda={lda} ldb={ldb}", flush=True)
    run_kernel(f"v{v}", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    rep = oracle.check(A, B, c.result(), rows=sample_rows(M, 16, seed=K))
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, rep


# Ragged products the plan gives to the persistent variant: its kernel on the whole tiles,
# then the right edge (all rows, the columns past the last whole tile column) and the bottom
# edge (the rows past the last whole tile row) as launches of their own, planned for their
# shapes. Every row of the bottom edge is checked with sampled rows elsewhere, each across all
# columns, so both edges are covered.
# The last case pads every row (A and B with NaN, C with guard cells; C's rows stay on 32-byte
# boundaries, which the plan asks of this kernel).
PS_EDGE_PLANS = [(8200, 8200, 128, 2, 0), (16383, 16384, 64, 1, 0), (4096 + 77, 4096, 96, 1, 0),
                 (8200, 8300, 96, 2, 1)]


@pytest.mark.parametrize("M,N,K,edges,padded", PS_EDGE_PLANS)
def test_persistent_plan_with_edges(gpu, M, N, K, edges, padded):
    lda, ldb, ldc = (K + 3, N + 5, N + 12) if padded else (K, N, N)
    plan = g.sgemm_f32_plan_describe(M, N, K, lda=lda, ldb=ldb, ldc=ldc)
    assert plan["name"] == "mfma_128x256x32_w2x4_ps" and plan["edge_launches"] == edges, plan
    rng = np.random.default_rng(M + 3 * N + 5 * K)
    A = wl.draw(rng, (M, K), "int")
    B = wl.draw(rng, (K, N), "int")
    _, dA, lda = device_matrix(A, lda)
    _, dB, ldb = device_matrix(B, ldb)
    c = GuardedC(M, N, ldc)
    print(f"[parity] {M}x{N}x{K} int auto (persistent, {edges} edge launches, "
          f"lda={lda} ldb={ldb} ldc={ldc})", flush=True)
    run_kernel("auto", M, N, K, dA, lda, dB, ldb, c)
    gpu.cuda.synchronize()
    rows = sorted(set(sample_rows(M, 16, seed=K) or []) | set(range(M // 128 * 128, M)))
    rep = oracle.check(A, B, c.result(), rows=rows)
    assert rep["n_nonfinite"] == 0 and rep["n_inexact"] == 0, rep


# large shapes whose tile counts fall just past a whole round of 256 x 256 tiles
STREAMK_PLAN_SHAPES = [(4500, 4500, 8192), (5000, 5000, 2048)]


def test_plan_covers_every_planned_variant(gpu):
    """The shapes above, with the five workloads, reach every variant the plan can pick:
    through the plain product's plan, or through the stream-K entry's plan (the 8-wave
    256 x 256 variant is planned for its stream-K form)."""
    shapes = AT_SCALE + [(w.M, w.N, w.K) for w in wl.WORKLOADS.values()]
    picked = {g.sgemm_f32_plan_describe(*s)["name"] for s in shapes}
    for s in shapes + STREAMK_PLAN_SHAPES:
        d = g.sgemm_f32_streamk_describe(*s)
        if d["streamk"]:
            picked.add(d["name"])
    planned = {g.variant_names()[i] for i in g.planned_variants()}
    assert planned <= picked, planned - picked
