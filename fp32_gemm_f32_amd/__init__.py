"""Python binding of the MI355X FP32 GEMM library (libsgemm_f32.so).

Argument marshalling only: every call goes straight to the C ABI of include/sgemm_f32.h,
and every step of the product runs in the library's HIP kernels. There is no fallback:
if the library is not built, importing the binding's functions raises.

Raw layer (same names and arguments as the C ABI; pointers are integers):
    sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0)
    sgemm_f32_naive(...), sgemm_f32_tiled(..., tile=32, pad=0, stream=0)
    sgemm_f32_splitk(..., splits, workspace, workspace_bytes, stream=0)
    sgemm_f32_splitk_workspace_size(M, N, K, splits) -> int
    sgemm_f32_streamk(..., variant, workspace, workspace_bytes, stream=0)
    sgemm_f32_streamk_workspace_size(M, N, K, lda, ldb, ldc, variant=-1) -> int
    sgemm_f32_streamk_noalloc(..., variant, stream=0)
    sgemm_f32_streamk_noalloc_scratch_bytes() -> int
    sgemm_f32_streamk_describe(M, N, K, variant=-1, num_cus=0) -> dict
    sgemm_f32_regtiled(..., tm=4, tn=4, stream=0)
    sgemm_f32_lds_transpose(rows, cols, src, ldi, dst, ldo, tile=32, pad=0, stream=0)
    sgemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=0)
    sgemm_f32_plan_describe(M, N, K, A, lda, B, ldb, C, ldc, num_cus=0) -> dict
    sgemm_f32_variant_describe(variant, M, N, K, lda, ldb, ldc, num_cus=0) -> dict
    sgemm_f32_variant_info(variant) -> dict, planned_variants() -> [index],
    streamk_variants() -> [index]
Tensor layer (torch tensors on the GPU, launched on torch's current stream):
    matmul(A, B, out=None, kernel="auto", variant=-1) -> C
"""
from __future__ import annotations

import ctypes
import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsgemm_f32.so")

SGEMM_OK = 0
STATUS_NAMES = {0: "SGEMM_OK", -1: "SGEMM_EINVAL_DIM", -2: "SGEMM_EINVAL_LD",
                -3: "SGEMM_EINVAL_PTR", -4: "SGEMM_EALIAS", -5: "SGEMM_ELAUNCH",
                -6: "SGEMM_EINVAL_ARG", -7: "SGEMM_ETOO_LARGE", -8: "SGEMM_ESCRATCH"}

_lib = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _load().sgemm_f32_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m fp32_gemm_f32_amd.build` "
                               "(or __graft_entry__.build()) first")
        # torch carries its own HIP runtime under the same soname as the system's. Loaded
        # first, it is the one the library binds to; loaded after the library, it would be a
        # second runtime in the process, and the library's own would see no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        i, p = ctypes.c_int, ctypes.c_void_p
        gemm = [i, i, i, p, i, p, i, p, i]
        lib.sgemm_f32.argtypes = gemm + [p]
        lib.sgemm_f32.restype = i
        lib.sgemm_f32_naive.argtypes = gemm + [p]
        lib.sgemm_f32_naive.restype = i
        lib.sgemm_f32_tiled.argtypes = gemm + [i, i, p]
        lib.sgemm_f32_tiled.restype = i
        lib.sgemm_f32_splitk.argtypes = gemm + [i, p, ctypes.c_size_t, p]
        lib.sgemm_f32_splitk.restype = i
        lib.sgemm_f32_splitk_workspace_size.argtypes = [i, i, i, i]
        lib.sgemm_f32_splitk_workspace_size.restype = ctypes.c_size_t
        lib.sgemm_f32_streamk.argtypes = gemm + [i, p, ctypes.c_size_t, p]
        lib.sgemm_f32_streamk.restype = i
        lib.sgemm_f32_streamk_workspace_size.argtypes = [i, i, i, i, i, i, i]
        lib.sgemm_f32_streamk_workspace_size.restype = ctypes.c_size_t
        lib.sgemm_f32_streamk_noalloc.argtypes = gemm + [i, p]
        lib.sgemm_f32_streamk_noalloc.restype = i
        lib.sgemm_f32_streamk_noalloc_scratch_bytes.argtypes = []
        lib.sgemm_f32_streamk_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.sgemm_f32_streamk_describe.argtypes = [i, i, i, i, i, ctypes.c_char_p, i]
        lib.sgemm_f32_streamk_describe.restype = i
        lib.sgemm_f32_regtiled.argtypes = gemm + [i, i, p]
        lib.sgemm_f32_regtiled.restype = i
        lib.sgemm_f32_lds_transpose.argtypes = [i, i, p, i, p, i, i, i, p]
        lib.sgemm_f32_lds_transpose.restype = i
        lib.sgemm_f32_variant.argtypes = [i] + gemm + [p]
        lib.sgemm_f32_variant.restype = i
        lib.sgemm_f32_variant_count.argtypes = []
        lib.sgemm_f32_variant_count.restype = i
        lib.sgemm_f32_variant_name.argtypes = [i]
        lib.sgemm_f32_variant_name.restype = ctypes.c_char_p
        lib.sgemm_f32_variant_info.argtypes = [i, ctypes.c_char_p, i]
        lib.sgemm_f32_variant_info.restype = i
        lib.sgemm_f32_status_string.argtypes = [i]
        lib.sgemm_f32_status_string.restype = ctypes.c_char_p
        lib.sgemm_f32_plan_describe.argtypes = gemm + [i, ctypes.c_char_p, i]
        lib.sgemm_f32_plan_describe.restype = i
        lib.sgemm_f32_variant_describe.argtypes = [i] * 8 + [ctypes.c_char_p, i]
        lib.sgemm_f32_variant_describe.restype = i
        lib.sgemm_f32_abi_version.argtypes = []
        lib.sgemm_f32_abi_version.restype = i
        _lib = lib
    return _lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(rc: int, where: str) -> None:
    if rc != SGEMM_OK:
        raise SgemmError(rc, where)


# ------------------------------------------------------------------ raw C-ABI layer -------

def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> None:
    _check(_load().sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream or None), "sgemm_f32")


def sgemm_f32_naive(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> None:
    _check(_load().sgemm_f32_naive(M, N, K, A, lda, B, ldb, C, ldc, stream or None),
           "sgemm_f32_naive")


def sgemm_f32_tiled(M, N, K, A, lda, B, ldb, C, ldc, tile=32, pad=0, stream=0) -> None:
    _check(_load().sgemm_f32_tiled(M, N, K, A, lda, B, ldb, C, ldc, tile, pad, stream or None),
           "sgemm_f32_tiled")


def sgemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_bytes,
                     stream=0) -> None:
    _check(_load().sgemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace or None,
                                    workspace_bytes, stream or None), "sgemm_f32_splitk")


def sgemm_f32_splitk_workspace_size(M, N, K, splits) -> int:
    return _load().sgemm_f32_splitk_workspace_size(M, N, K, splits)


def sgemm_f32_streamk(M, N, K, A, lda, B, ldb, C, ldc, variant, workspace, workspace_bytes,
                      stream=0) -> None:
    _check(_load().sgemm_f32_streamk(M, N, K, A, lda, B, ldb, C, ldc, variant,
                                     workspace or None, workspace_bytes, stream or None),
           "sgemm_f32_streamk")


def sgemm_f32_streamk_workspace_size(M, N, K, lda=None, ldb=None, ldc=None, variant=-1) -> int:
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return _load().sgemm_f32_streamk_workspace_size(M, N, K, lda, ldb, ldc, variant)


def sgemm_f32_streamk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, variant=-1, stream=0) -> None:
    _check(_load().sgemm_f32_streamk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, variant,
                                             stream or None), "sgemm_f32_streamk_noalloc")


def sgemm_f32_streamk_noalloc_scratch_bytes() -> int:
    return _load().sgemm_f32_streamk_noalloc_scratch_bytes()


def sgemm_f32_streamk_describe(M, N, K, variant=-1, num_cus=0) -> dict:
    buf = ctypes.create_string_buffer(1024)
    rc = _load().sgemm_f32_streamk_describe(M, N, K, variant, num_cus, buf, len(buf))
    if rc < 0:
        raise SgemmError(rc, "sgemm_f32_streamk_describe")
    return json.loads(buf.value.decode())


def sgemm_f32_regtiled(M, N, K, A, lda, B, ldb, C, ldc, tm=4, tn=4, stream=0) -> None:
    _check(_load().sgemm_f32_regtiled(M, N, K, A, lda, B, ldb, C, ldc, tm, tn, stream or None),
           "sgemm_f32_regtiled")


def sgemm_f32_lds_transpose(rows, cols, src, ldi, dst, ldo, tile=32, pad=0, stream=0) -> None:
    _check(_load().sgemm_f32_lds_transpose(rows, cols, src, ldi, dst, ldo, tile, pad,
                                           stream or None), "sgemm_f32_lds_transpose")


def sgemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> None:
    _check(_load().sgemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream or None),
           "sgemm_f32_variant")


def variant_names() -> list[str]:
    lib = _load()
    return [lib.sgemm_f32_variant_name(i).decode() for i in range(lib.sgemm_f32_variant_count())]


def sgemm_f32_variant_info(variant) -> dict:
    buf = ctypes.create_string_buffer(1024)
    rc = _load().sgemm_f32_variant_info(variant, buf, len(buf))
    if rc < 0:
        raise SgemmError(rc, "sgemm_f32_variant_info")
    return json.loads(buf.value.decode())


def planned_variants() -> list[int]:
    """Indices of the variants the automatic plan may pick."""
    return [i for i in range(len(variant_names())) if sgemm_f32_variant_info(i)["planned"]]


def streamk_variants() -> list[int]:
    """Indices of the variants with a stream-K form (those sgemm_f32_streamk accepts)."""
    return [i for i in range(len(variant_names())) if sgemm_f32_variant_info(i)["streamk"]]


def sgemm_f32_plan_describe(M, N, K, A=0, lda=None, B=0, ldb=None, C=0, ldc=None,
                            num_cus=0) -> dict:
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    buf = ctypes.create_string_buffer(1024)
    rc = _load().sgemm_f32_plan_describe(M, N, K, A or None, lda, B or None, ldb, C or None,
                                         ldc, num_cus, buf, len(buf))
    if rc < 0:
        raise SgemmError(rc, "sgemm_f32_plan_describe")
    return json.loads(buf.value.decode())


def sgemm_f32_variant_describe(variant, M, N, K, lda=None, ldb=None, ldc=None,
                               num_cus=0) -> dict:
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    buf = ctypes.create_string_buffer(1024)
    rc = _load().sgemm_f32_variant_describe(variant, M, N, K, lda, ldb, ldc, num_cus, buf,
                                            len(buf))
    if rc < 0:
        raise SgemmError(rc, "sgemm_f32_variant_describe")
    return json.loads(buf.value.decode())


def abi_version() -> int:
    return _load().sgemm_f32_abi_version()


# ------------------------------------------------------------------ tensor layer ----------

def _ld(t) -> int:
    """Leading dimension of a row-major 2-D tensor with unit column stride."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("columns must be contiguous (row-major, unit column stride)")
    return max(t.stride(0), t.shape[1], 1)


def matmul(A, B, out=None, kernel: str = "auto", variant: int = -1, tile=32, pad: int = 0):
    """C = A x B for float32 CUDA/HIP tensors, on torch's current stream.

    kernel: "auto" (the hot path, or the given variant), "naive", "tiled", "regtiled"
    (tile = (tm, tn)), "splitk" (variant = number of splits, -1 for automatic) or
    "streamk" (variant = tile variant forced into stream-K, -1 for the automatic choice
    between the plain and the stream-K form). The split-K and stream-K workspaces are
    torch allocations made here.
    """
    import torch

    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise TypeError("A and B must be float32")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or out.device != A.device:
        raise ValueError("out must be a float32 (M, N) tensor on A's device")
    stream = torch.cuda.current_stream(A.device).cuda_stream
    args = (M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), out.data_ptr(), _ld(out))
    with torch.cuda.device(A.device):
        if kernel == "auto":
            if variant < 0:
                sgemm_f32(*args, stream=stream)
            else:
                sgemm_f32_variant(variant, *args, stream=stream)
        elif kernel == "naive":
            sgemm_f32_naive(*args, stream=stream)
        elif kernel == "tiled":
            sgemm_f32_tiled(*args, tile=tile, pad=pad, stream=stream)
        elif kernel == "splitk":
            splits = variant if variant >= 0 else 0
            ws_bytes = sgemm_f32_splitk_workspace_size(M, N, K, splits)
            ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=A.device)
            sgemm_f32_splitk(*args, splits, ws.data_ptr(), ws_bytes, stream=stream)
        elif kernel == "streamk":
            ws_bytes = sgemm_f32_streamk_workspace_size(M, N, K, args[4], args[6], args[8],
                                                        variant)
            ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=A.device)
            sgemm_f32_streamk(*args, variant, ws.data_ptr(), ws_bytes, stream=stream)
        elif kernel == "regtiled":
            tm, tn = tile if isinstance(tile, tuple) else (4, 4)
            sgemm_f32_regtiled(*args, tm=tm, tn=tn, stream=stream)
        else:
            raise ValueError(f"unknown kernel {kernel!r}")
    return out
