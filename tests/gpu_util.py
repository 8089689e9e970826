"""Helpers for the GPU tests: device operands with padded rows and guard bands, and the
call into the C ABI for each kernel under test. Expected values come from the oracle
only (oracle.check on the host copy)."""
from __future__ import annotations

import numpy as np

import fp32_gemm_f32_amd as g

SENTINEL = np.float32(-12345.5)   # guard-band value: must survive every call bit for bit
TOL = 1e-5                        # max |C - C_ref| / sum_k |a_ik b_kj| on float inputs


def torch_mod():
    import torch
    return torch


def device_matrix(host: np.ndarray, ld: int | None = None, pad=np.nan, offset: int = 0):
    """Copy a row-major host matrix into a device buffer of rows of `ld` floats whose extra
    columns hold `pad`; `offset` floats are skipped at the front (misaligned base).
    Returns (buffer, view, ld)."""
    torch = torch_mod()
    rows, cols = host.shape
    ld = cols if ld is None else ld
    buf = np.full(offset + max(rows * ld, 1), pad, dtype=np.float32)
    if rows and cols:
        buf[offset:offset + rows * ld].reshape(rows, ld)[:, :cols] = host
    dev = torch.from_numpy(buf).to("cuda")
    view = dev[offset:offset + rows * ld].view(rows, ld)[:, :cols] if rows * ld else dev[:0]
    return dev, view, ld


class GuardedC:
    """C inside a buffer with one guard row above and below and ldc - N guard columns,
    all set to SENTINEL; C itself is pre-filled with NaN so unwritten cells show."""

    def __init__(self, M: int, N: int, ldc: int | None = None, offset: int = 0):
        torch = torch_mod()
        self.M, self.N = M, N
        self.ldc = N if ldc is None else ldc
        self.offset = offset
        total = offset + (M + 2) * self.ldc
        host = np.full(total, SENTINEL, dtype=np.float32)
        host[offset + self.ldc: offset + (M + 1) * self.ldc].reshape(M, self.ldc)[:, :N] = np.nan
        self.host_init = host
        self.dev = torch.from_numpy(host.copy()).to("cuda")

    @property
    def ptr(self) -> int:
        return self.dev.data_ptr() + 4 * (self.offset + self.ldc)

    def result(self) -> np.ndarray:
        """The M x N result (host copy); asserts the guard cells are untouched."""
        out = self.dev.cpu().numpy()
        lo, hi = self.offset + self.ldc, self.offset + (self.M + 1) * self.ldc
        body = out[lo:hi].reshape(self.M, self.ldc)[:, :self.N]
        outside = np.ones(out.size, dtype=bool)
        outside[lo:hi].reshape(self.M, self.ldc)[:, :self.N] = False
        assert (out[outside].view(np.uint32) == SENTINEL.view(np.uint32)).all(), \
            "a cell outside C's M x N region was written"
        return body


def run_kernel(kernel: str, M, N, K, A_view, lda, B_view, ldb, c: GuardedC, stream=0):
    """Call one entry point of the C ABI. kernel: auto | naive | tiled16 | tiled32 |
    tiled32p | v<index>."""
    args = (M, N, K, A_view.data_ptr(), lda, B_view.data_ptr(), ldb, c.ptr, c.ldc)
    if kernel == "auto":
        g.sgemm_f32(*args, stream=stream)
    elif kernel == "naive":
        g.sgemm_f32_naive(*args, stream=stream)
    elif kernel.startswith("tiled"):
        tile = int(kernel[5:7])
        g.sgemm_f32_tiled(*args, tile=tile, pad=1 if kernel.endswith("p") else 0, stream=stream)
    elif kernel.startswith("v"):
        g.sgemm_f32_variant(int(kernel[1:]), *args, stream=stream)
    else:
        raise ValueError(kernel)


def all_variants():
    return list(range(len(g.variant_names())))
