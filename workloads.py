"""Seeded synthetic operands for C = A x B, shared by the tests and the benchmark.

This module holds no GEMM arithmetic: it only draws operand matrices. Every draw is
numpy's PCG64 (np.random.default_rng(seed)) in float64, then rounded to float32, so
the same (config, variant) gives the same bits on every machine.

The five workloads follow the shapes the pages work through (6 x 6 x 9 from the tiling
visualiser's controls, N = 1024 from the memory-hierarchy walkthrough) plus a ragged
shape, the large square headline shape and a low-K shape:

  name  M      N      K     distribution
  c1    6      6      9     uniform[-1, 1]    (integer variant: uniform in {-4..4})
  c2    1024   1024   1024  uniform[-1, 1]
  c3    1023   1025   1027  standard normal
  c4    8192   8192   8192  uniform[-1, 1]
  c5    16384  16384  64    uniform[-1, 1]
  sk    256    256    32768 uniform[-1, 1]    (an under-filled shape for split-K)
  rk    4500   4500   8192  uniform[-1, 1]    (a large ragged shape for stream-K)

Seeds: A = 1000*i + 1, B = 1000*i + 2 for config ci; the integer variant uses
1000*i + 3 and 1000*i + 4. All operands are packed row-major (lda = K, ldb = N).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    M: int
    N: int
    K: int
    dist: str          # "uniform" (U[-1,1]) or "normal" (N(0,1))
    label: str

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> str:
        return f"{self.name} {self.M}x{self.N}x{self.K} {self.dist}"


WORKLOADS = {
    "c1": Workload("c1", 1, 6, 6, 9, "uniform", "worked example 6x6x9"),
    "c2": Workload("c2", 2, 1024, 1024, 1024, "uniform", "square 1024^3"),
    "c3": Workload("c3", 3, 1023, 1025, 1027, "normal", "ragged 1023x1025x1027"),
    "c4": Workload("c4", 4, 8192, 8192, 8192, "uniform", "square 8192^3"),
    "c5": Workload("c5", 5, 16384, 16384, 64, "uniform", "low-K 16384x16384x64"),
    # not one of the five: an under-filled shape (16 tiles of 64 x 64) for split-K
    "sk": Workload("sk", 6, 256, 256, 32768, "uniform", "under-filled 256x256x32768"),
    # not one of the five: 18 x 18 tiles of 256 x 256, just past one round of 256 compute
    # units, so whole-tile rounds leave most units idle in the last one (stream-K's case)
    "rk": Workload("rk", 7, 4500, 4500, 8192, "uniform", "ragged large 4500x4500x8192"),
}


def draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """One float32 matrix of the named distribution."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "int":
        x = rng.integers(-4, 5, size=shape).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(x.astype(np.float32))


def operands(name: str, variant: str = "float") -> tuple[np.ndarray, np.ndarray]:
    """(A, B) for a named workload; variant "float" (its own distribution) or "int"."""
    w = WORKLOADS[name]
    if variant == "float":
        sa, sb, dist = 1000 * w.index + 1, 1000 * w.index + 2, w.dist
    elif variant == "int":
        sa, sb, dist = 1000 * w.index + 3, 1000 * w.index + 4, "int"
    else:
        raise ValueError(f"unknown variant {variant!r}")
    A = draw(np.random.default_rng(sa), (w.M, w.K), dist)
    B = draw(np.random.default_rng(sb), (w.K, w.N), dist)
    return A, B


def random_operands(M: int, N: int, K: int, seed: int, dist: str = "uniform",
                    lda: int | None = None, ldb: int | None = None,
                    pad_value: float = float("nan")):
    """(A, B) of the given shape, optionally embedded in wider row-major buffers.

    With lda > K (ldb > N) the returned A (B) is a view of an M x lda (K x ldb) array
    whose extra columns hold pad_value (NaN by default), so a kernel that reads past the
    logical edge makes the result non-finite.
    """
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), dist)
    B = draw(rng, (K, N), dist)
    if lda is not None and lda != K:
        if lda < K:
            raise ValueError("lda < K")
        buf = np.full((M, lda), pad_value, dtype=np.float32)
        buf[:, :K] = A
        A = buf[:, :K]
    if ldb is not None and ldb != N:
        if ldb < N:
            raise ValueError("ldb < N")
        buf = np.full((K, ldb), pad_value, dtype=np.float32)
        buf[:, :N] = B
        B = buf[:, :N]
    return A, B
