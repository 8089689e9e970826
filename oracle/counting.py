"""The pages' memory-traffic model, as an instrumented simulation plus its closed forms.

TEST INFRASTRUCTURE ONLY (same rule as the rest of oracle/).

The pages count element reads rather than bytes or cache lines:
  * "SGEMM: Shared Memory Tiling Visualizer", "Why Tiling Works (The Math)": the naive
    kernel launches one thread per C element and each thread reads one A and one B value
    per k step, so it makes 2*M*N*K global reads; with cooperative tiles reused TILE_SIZE
    times the ideal count is 2*M*N*K / TILE_SIZE.
  * "Visual walkthrough - Memory hierarchy", Steps 1-5: the same counts at N = 1024 and
    T = 16 (2N reads per thread, N^2 threads, N/T tiles, a T-fold reduction).
  * "SGEMM: 2D Register Tiling Visualizer", "Why 2D Register Tiling Dominates": per inner
    step a thread makes TM + TN shared reads and TM * TN FMAs.
  * "Shared Memory Tiling", "The reuse argument" and "Choosing a tile size": intensity
    0.25 FLOP/byte naive, times TILE when tiled; shared bytes 2 * TILE * (TILE + pad) * 4.

Readings where the pages are silent or garbled (each is listed in the design notes):
  * the tile-loop bound is the ceiling ceil(K / T): the printed integer division would
    drop the last partial tile;
  * a masked load (the `cond ? load : 0` form of the visualiser's code panel) reads global
    memory only when its condition holds, so only in-bounds loads are counted;
  * a thread whose output lies outside C still runs the shared-memory loop (the printed
    kernel has no early exit), so its shared reads are counted.
"""
from __future__ import annotations

from dataclasses import dataclass


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Counts:
    global_reads: int = 0   # element reads from global memory
    shared_reads: int = 0   # element reads from shared memory
    fmas: int = 0           # multiply-adds issued (in-bounds or not)
    threads: int = 0        # threads launched
    blocks: int = 0         # blocks launched


# ---------------------------------------------------------------- simulations --------------

def simulate_naive(M: int, N: int, K: int) -> Counts:
    """Run the one-thread-per-output kernel thread by thread, counting its reads."""
    c = Counts()
    for _row in range(M):
        for _col in range(N):
            c.threads += 1
            for _k in range(K):
                c.global_reads += 1   # A[row][k]
                c.global_reads += 1   # B[k][col]
                c.fmas += 1
    c.blocks = 1 if M * N else 0
    return c


def simulate_tiled(M: int, N: int, K: int, T: int) -> Counts:
    """Run the masked shared-memory tiled kernel block by block, thread by thread.

    Grid ceil(N/T) x ceil(M/T) blocks of T x T threads; per tile index each thread loads
    tileA[ty][tx] (if row < M and its k < K) and tileB[ty][tx] (if its k < K and col < N),
    then reads T values of each tile from shared memory.
    """
    c = Counts()
    n_tiles = _ceil(K, T)
    for by in range(_ceil(M, T)):
        for bx in range(_ceil(N, T)):
            c.blocks += 1
            for ty in range(T):
                for tx in range(T):
                    c.threads += 1
                    row = by * T + ty
                    col = bx * T + tx
                    for t in range(n_tiles):
                        col_a = t * T + tx
                        row_b = t * T + ty
                        if row < M and col_a < K:
                            c.global_reads += 1
                        if row_b < K and col < N:
                            c.global_reads += 1
                        for _k in range(T):
                            c.shared_reads += 2
                            c.fmas += 1
    return c


def simulate_register_tiled(M: int, N: int, K: int, BM: int, BN: int, BK: int,
                            TM: int, TN: int) -> Counts:
    """Run the 2-D register-tiled (outer product) kernel block by block.

    Each block owns a BM x BN tile of C with (BM/TM)*(BN/TN) threads; per K step of BK
    the block cooperatively loads the in-bounds part of a BM x BK tile of A and a
    BK x BN tile of B; per inner step each thread loads TM values of A and TN of B into
    registers and does TM*TN multiply-adds.
    """
    if BM % TM or BN % TN:
        raise ValueError("register tile must divide the block tile")
    c = Counts()
    threads_per_block = (BM // TM) * (BN // TN)
    for by in range(_ceil(M, BM)):
        for bx in range(_ceil(N, BN)):
            c.blocks += 1
            c.threads += threads_per_block
            for bk in range(0, K, BK):
                for r in range(BM):
                    for kk in range(BK):
                        if by * BM + r < M and bk + kk < K:
                            c.global_reads += 1
                for kk in range(BK):
                    for j in range(BN):
                        if bk + kk < K and bx * BN + j < N:
                            c.global_reads += 1
                for _thread in range(threads_per_block):
                    for _dot in range(BK):
                        for _i in range(TM):
                            c.shared_reads += 1
                        for _j in range(TN):
                            c.shared_reads += 1
                        for _i in range(TM):
                            for _j in range(TN):
                                c.fmas += 1
    return c


# ---------------------------------------------------------------- closed forms -------------

def naive_reads(M: int, N: int, K: int) -> int:
    """M*N threads times 2K reads each."""
    return 2 * M * N * K


def tiled_reads_ideal(M: int, N: int, K: int, T: int) -> float:
    """The pages' ideal count, 2MNK / T (exact when T divides M and N)."""
    return 2 * M * N * K / T


def tiled_reads_exact(M: int, N: int, K: int, T: int) -> int:
    """In-bounds loads of the masked tiled kernel: each A element is loaded once per
    block column, each B element once per block row."""
    return M * K * _ceil(N, T) + K * N * _ceil(M, T)


def block_tiled_bytes(M: int, N: int, K: int, BM: int, BN: int, elem_bytes: int = 4) -> int:
    """Operand bytes a BM x BN block-tiled GEMM requests from memory (no cache reuse)."""
    return elem_bytes * (M * K * _ceil(N, BN) + K * N * _ceil(M, BM))


def compulsory_bytes(M: int, N: int, K: int, elem_bytes: int = 4) -> int:
    """Read A and B once, write C once."""
    return elem_bytes * (M * K + K * N + M * N)


def intensity_naive(elem_bytes: int = 4) -> float:
    """FLOP per byte of a length-N dot product with no reuse: 2N FLOP over 2N elements."""
    n = 1
    return (2 * n) / (2 * n * elem_bytes)


def intensity_tiled(T: int, elem_bytes: int = 4) -> float:
    """Each element read from memory backs T multiply-adds instead of one."""
    return intensity_naive(elem_bytes) * T


def shared_reads_per_fma(TM: int, TN: int) -> tuple[int, int]:
    """(shared reads, FMAs) per inner step of a TM x TN register tile."""
    return TM + TN, TM * TN


def shared_bytes_per_block(T: int, pad: int = 0, elem_bytes: int = 4) -> int:
    """Two T x (T + pad) FP32 tiles."""
    return 2 * T * (T + pad) * elem_bytes
