"""The pages' read-count model: the instrumented simulation of each kernel the pages
describe must agree with the closed forms, and both with every number the pages print
(tests/golden/page_counts.json names the page and section of each)."""
import json
import os

import pytest

from oracle import counting as cm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_counts.json")))
G = {e["id"]: e for e in GOLDEN["entries"]}


def test_tiled_example_128():
    e = G["tiled_ideal_example"]
    M, N, K, T = e["M"], e["N"], e["K"], e["T"]
    assert cm.tiled_reads_ideal(M, N, K, T) == e["tiled_reads_ideal"]
    sim = cm.simulate_tiled(M, N, K, T)
    assert sim.global_reads == e["tiled_reads_ideal"] == cm.tiled_reads_exact(M, N, K, T)


def test_walkthrough_counts():
    n = G["naive_per_thread"]["N"]
    assert 2 * n == G["naive_per_thread"]["reads_per_thread"]
    assert n * n == G["naive_threads"]["threads"]
    total = cm.naive_reads(n, n, n)
    assert total == G["naive_threads"]["threads"] * G["naive_per_thread"]["reads_per_thread"]
    assert round(total / 1e9, 2) == G["naive_total"]["naive_reads_rounded_billions"]
    T = G["tiles_along_k"]["T"]
    assert n // T == G["tiles_along_k"]["tiles"]
    assert cm.tiled_reads_ideal(n, n, n, T) == G["tiled_total"]["tiled_reads"]
    assert cm.tiled_reads_exact(n, n, n, T) == G["tiled_total"]["tiled_reads"]
    assert total / cm.tiled_reads_exact(n, n, n, T) == G["reduction_factor"]["ratio"]


def test_no_gain_at_tile_one():
    T = G["no_gain_at_T1"]["T"]
    for (M, N, K) in [(4, 4, 8), (6, 6, 9), (3, 5, 2)]:
        sim = cm.simulate_tiled(M, N, K, T)
        assert cm.naive_reads(M, N, K) / sim.global_reads == G["no_gain_at_T1"]["ratio"]


@pytest.mark.parametrize("M,N,K", [(6, 6, 9), (4, 4, 8), (5, 3, 7), (1, 1, 1), (2, 9, 4)])
def test_naive_simulation(M, N, K):
    sim = cm.simulate_naive(M, N, K)
    assert sim.global_reads == cm.naive_reads(M, N, K)
    assert sim.threads == M * N and sim.fmas == M * N * K


@pytest.mark.parametrize("M,N,K,T", [(4, 4, 8, 2), (6, 6, 9, 3), (6, 6, 9, 2), (8, 8, 8, 4),
                                     (5, 7, 3, 2), (7, 5, 11, 4), (1, 1, 1, 3)])
def test_tiled_simulation_exact_form(M, N, K, T):
    sim = cm.simulate_tiled(M, N, K, T)
    assert sim.global_reads == cm.tiled_reads_exact(M, N, K, T)
    if M % T == 0 and N % T == 0:
        assert sim.global_reads == cm.tiled_reads_ideal(M, N, K, T)
    # every launched thread runs the shared loop over ceil(K/T) tiles
    assert sim.shared_reads == sim.threads * 2 * T * (-(-K // T))


def test_worked_shape_6x6x9():
    # the visualiser's problem size: with its TILE=3 everything divides except nothing
    assert cm.simulate_tiled(6, 6, 9, 3).global_reads == 216
    # with the code panel's TILE_SIZE=2, K=9 leaves a partial last tile
    assert cm.simulate_tiled(6, 6, 9, 2).global_reads == 324


def test_register_tiled_example():
    # 8x8 times 8x8 with BM=BN=BK=4, TM=TN=2 (the register-tiling visualiser's setup)
    sim = cm.simulate_register_tiled(8, 8, 8, 4, 4, 4, 2, 2)
    assert sim.blocks == 4 and sim.threads == 16
    assert sim.global_reads == cm.tiled_reads_exact(8, 8, 8, 4) == 256
    assert sim.fmas == 8 * 8 * 8
    assert sim.shared_reads == 512
    sr, f = cm.shared_reads_per_fma(2, 2)
    assert sim.shared_reads / sim.fmas == sr / f


@pytest.mark.parametrize("key", ["strip_1d", "square_2d_4", "square_2d_8"])
def test_shared_to_fma_ratios(key):
    e = G[key]
    assert cm.shared_reads_per_fma(e["TM"], e["TN"]) == (e["shared_reads"], e["fmas"])
    # the simulation reproduces the per-step ratio
    sim = cm.simulate_register_tiled(e["TM"], e["TN"], 1, e["TM"], e["TN"], 1, e["TM"], e["TN"])
    assert (sim.shared_reads, sim.fmas) == (e["shared_reads"], e["fmas"])
    if "fmas_per_shared_read" in e:
        assert e["fmas"] / e["shared_reads"] == e["fmas_per_shared_read"]


def test_intensity():
    assert cm.intensity_naive() == G["intensity_naive"]["flop_per_byte"]
    assert cm.intensity_tiled(G["intensity_tiled"]["TILE"]) == G["intensity_tiled"]["flop_per_byte"]
    # the naive figure from counts: 2 FLOP per k against 2 elements of 4 bytes
    sim = cm.simulate_naive(3, 3, 5)
    assert (2 * sim.fmas) / (4 * sim.global_reads) == G["intensity_naive"]["flop_per_byte"]


@pytest.mark.parametrize("key", ["smem_tile16", "smem_tile32"])
def test_shared_bytes(key):
    e = G[key]
    assert cm.shared_bytes_per_block(e["TILE"], e["pad"]) == e["bytes"]


def test_block_tiled_bytes_reduce_to_tiled_count():
    # a square block tile of side T requests the same elements as the scalar T-tiled kernel
    for (M, N, K, T) in [(64, 64, 64, 16), (1023, 1025, 1027, 32), (6, 6, 9, 2)]:
        assert cm.block_tiled_bytes(M, N, K, T, T) == 4 * cm.tiled_reads_exact(M, N, K, T)
    assert cm.compulsory_bytes(8192, 8192, 8192) == 805306368
