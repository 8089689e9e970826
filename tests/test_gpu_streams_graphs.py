"""The C ABI under HIP graph capture and from several host threads at once.

Graph capture: the hot path launches kernels only (no memset, no allocation, no host
synchronisation), so a captured call replays correctly, as do split-K's two kernels and
stream-K's main and fixup kernels; every replay is checked against the oracle, with eager
work and synchronisation between replays.
Threads: the library keeps no mutable state beyond a per-device CU-count cache, so four host
threads, each on its own stream, get correct results at the same time."""
import threading

import numpy as np
import pytest

import fp32_gemm_f32_amd as g
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.library()
    return torch


def int_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    return wl.draw(rng, (M, K), "int"), wl.draw(rng, (K, N), "int")


@pytest.mark.parametrize("M,N,K,kernel", [(1000, 700, 300, "auto"), (257, 259, 1031, "auto"),
                                          (256, 256, 8192, "splitk"), (64, 96, 0, "auto"),
                                          (1023, 1025, 1027, "streamk"),
                                          (256, 256, 8192, "streamk")])
def test_graph_capture_and_replay(gpu, M, N, K, kernel):
    torch = gpu
    A, B = int_operands(M, N, K, M + N + K)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.full((M, N), float("nan"), device="cuda")
    ws = None
    if kernel == "splitk":
        ws_bytes = g.sgemm_f32_splitk_workspace_size(M, N, K, 4)
        ws = torch.empty(ws_bytes // 4, device="cuda")
    sk_variant = -1
    if kernel == "streamk":
        # the 64 x 64 tile with two workgroups per CU shares tiles on both shapes
        sk_variant = g.variant_names().index("mfma_64x64x32_w2x1_kg2_dl")
        ws_bytes = g.sgemm_f32_streamk_workspace_size(M, N, K, variant=sk_variant)
        assert ws_bytes > 0 and g.sgemm_f32_streamk_describe(M, N, K, sk_variant)["streamk"]
        ws = torch.empty(ws_bytes // 4, device="cuda")
    args = (M, N, K, dA.data_ptr(), max(K, 1), dB.data_ptr(), N, dC.data_ptr(), N)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    print(f"[graph] {M}x{N}x{K} {kernel} capture", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            s = torch.cuda.current_stream().cuda_stream
            if kernel == "splitk":
                g.sgemm_f32_splitk(*args, 4, ws.data_ptr(), ws.numel() * 4, stream=s)
            elif kernel == "streamk":
                g.sgemm_f32_streamk(*args, sk_variant, ws.data_ptr(), ws.numel() * 4, stream=s)
            else:
                g.sgemm_f32(*args, stream=s)
    torch.cuda.synchronize()
    for replay in range(4):
        dC.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        if K == 0:   # the empty sum
            assert (C == 0).all(), replay
            continue
        rep = oracle.check(A, B, C)
        assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, (replay, rep)


def test_threads_with_own_streams(gpu):
    torch = gpu
    shapes = [(700, 900, 513), (1024, 1024, 1024), (333, 1500, 77), (2048, 256, 4096)]
    results = [None] * len(shapes)
    errors = []

    def work(i, M, N, K):
        try:
            A, B = int_operands(M, N, K, 100 + i)
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                dA = torch.from_numpy(A).cuda()
                dB = torch.from_numpy(B).cuda()
                for _ in range(5):
                    dC = g.matmul(dA, dB)
                stream.synchronize()
                results[i] = (A, B, dC.cpu().numpy())
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    print("[threads] 4 threads x 5 calls", flush=True)
    threads = [threading.Thread(target=work, args=(i, *s)) for i, s in enumerate(shapes)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i, (A, B, C) in enumerate(results):
        rep = oracle.check(A, B, C)
        assert rep["n_inexact"] == 0 and rep["n_nonfinite"] == 0, (shapes[i], rep)
