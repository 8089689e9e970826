#!/usr/bin/env python3
"""Throughput of the hot path on one MI355X: FP32 C = A x B through the C ABI's sgemm_f32.

One step is one call of sgemm_f32 over the whole workload (the default is the square
8192^3 product with A, B ~ U[-1, 1], packed row-major). Inputs are drawn on the host from
fixed seeds, copied to HBM, and are resident before timing starts. W untimed steps, then
exactly K timed steps between two device synchronisations, timed with HIP events recorded
on the stream the kernels are launched on (torch's current stream).

Prints one JSON line on stdout:
  value        whole-job GFLOP/s = 2 M N K * steps / elapsed
  roofline     the kernel's achieved TFLOP/s (algorithmic 2MNK per launch / average
               launch time) against the MI355X FP32 matrix peak; for a workload whose
               HBM floor is the larger one, GB/s of compulsory bytes against 8 TB/s.
               traffic = measured HBM bytes per launch from the committed rocprofv3
               counter summary, or null unless it was taken on the same gfx950 machine
               code of that kernel and the same tile variant as this run.
  cpu_baseline the CPU oracle (fp64 triple loop) timed on this host on a bounded sample
               of rows of the same product; the same rows of the GPU result are checked
               against it.
Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense FP32 matrix peak
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 78.6      # MI355X FP32 vector FMA without packed FP32
LIB_PATH = os.path.join(ROOT, "fp32_gemm_f32_amd", "libsgemm_f32.so")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _elf_sections(data: bytes) -> dict:
    """Section name -> (bytes, load address, index) of a little-endian ELF64 image (only what
    the hashes below need)."""
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    hdr = lambda i: struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)
    strtab = hdr(shstrndx)
    names = data[strtab[4]:strtab[4] + strtab[5]]
    out = {}
    for i in range(shnum):
        h = hdr(i)
        out[names[h[0]:names.index(b"\0", h[0])].decode()] = (data[h[4]:h[4] + h[5]], h[3], i)
    return out


def _gfx950_code_objects(lib_path: str):
    """The gfx950 device code objects inside the library's offload bundles, one bundle per
    translation unit (empty when the file is missing or is not such a library)."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    try:
        with open(lib_path, "rb") as f:
            fat = _elf_sections(f.read())[".hip_fatbin"][0]
    except (OSError, KeyError, struct.error, ValueError):
        return []
    out = []
    start = fat.find(magic)
    while start >= 0:
        n, = struct.unpack_from("<Q", fat, start + 24)
        off, end = start + 32, start + 32
        for _ in range(n):
            o, size, tlen = struct.unpack_from("<QQQ", fat, off)
            off += 24
            triple = fat[off:off + tlen].decode()
            off += tlen
            end = max(end, start + o + size)
            if "gfx950" in triple:
                out.append(fat[start + o:start + o + size])
        start = fat.find(magic, max(end, start + 1))
    return out


def kernel_symbols(lib_path: str = LIB_PATH) -> dict:
    """Mangled kernel name -> hash of its gfx950 machine code: the function's instructions
    and its kernel descriptor (registers, LDS, launch settings). Comments, asserts, other
    kernels and the build directory do not change a kernel's hash; any change to what that
    kernel executes does."""
    out = {}
    for co in _gfx950_code_objects(lib_path):
        secs = _elf_sections(co)
        by_index = {idx: (data, addr) for data, addr, idx in secs.values()}
        symtab, strtab = secs[".symtab"][0], secs[".strtab"][0]
        syms = {}
        for i in range(len(symtab) // 24):
            st_name, st_info, _, shndx, value, size = struct.unpack_from("<IBBHQQ", symtab, 24 * i)
            if shndx not in by_index or size == 0:
                continue
            name = strtab[st_name:strtab.index(b"\0", st_name)].decode()
            data, addr = by_index[shndx]
            syms[name] = data[value - addr:value - addr + size]
        for name, code in syms.items():
            kd = syms.get(name + ".kd")
            if kd is not None and len(kd) == 64:
                # bytes 16..23 of a kernel descriptor hold the distance from it to the code,
                # which moves when other kernels are added; everything else is the kernel's
                h = hashlib.sha256(code)
                h.update(kd[:16] + bytes(8) + kd[24:])
                out[name] = h.hexdigest()[:16]
    return out


def kernel_code_hash(symbol: str, lib_path: str = LIB_PATH):
    """Hash of one kernel's gfx950 machine code in the built library, or None when the
    library is not built or holds no such kernel."""
    return kernel_symbols(lib_path).get(symbol)


def measured_traffic(workload: str, variant: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    machine code of the kernel that runs now and on the variant the plan picks now."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if (not entry or entry.get("variant") != variant
            or kernel_code_hash(entry.get("kernel_symbol", "")) != entry.get("kernel_code_sha")
            or entry.get("kernel_code_sha") is None):
        return None
    return entry.get("bytes_per_launch")


def copy_calibration(mib: int, steps: int) -> None:
    """A plain device copy of a known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": steps}))


def cpu_baseline(A, B, C_dev, M, N, K, seconds: float):
    """Time the oracle on a bounded sample of rows and check the GPU's rows against it."""
    import numpy as np

    import oracle
    lib = oracle.load()
    rows_all = np.arange(M, dtype=np.int64)
    C_host = C_dev.cpu().numpy()
    # calibrate on two rows per thread, then size the sample to the time budget
    n_probe = min(len(rows_all), 2 * oracle.threads(lib))
    probe = rows_all[np.linspace(0, len(rows_all) - 1, num=n_probe).astype(np.int64)]
    t0 = time.perf_counter()
    oracle.check(A, B, C_host, rows=probe, lib=lib)
    t_probe = time.perf_counter() - t0
    per_row = max(t_probe / len(probe), 1e-6)
    n_rows = int(min(len(rows_all), max(len(probe), seconds / per_row)))
    rows = rows_all[np.linspace(0, len(rows_all) - 1, num=n_rows).astype(np.int64)]
    t0 = time.perf_counter()
    rep = oracle.check(A, B, C_host, rows=rows, lib=lib)
    t = time.perf_counter() - t0
    flop = 2.0 * len(rows) * N * K
    cores = oracle.threads(lib)
    # the same oracle on one thread, over a few of those rows (about 3 s of work)
    n1 = int(min(len(rows), max(1, 3.0 / (per_row * cores))))
    rows1 = rows[np.linspace(0, len(rows) - 1, num=n1).astype(np.int64)]
    prev = oracle.set_threads(1, lib)
    try:
        t0 = time.perf_counter()
        oracle.check(A, B, C_host, rows=rows1, lib=lib)
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(prev, lib)
    return {"value": round(flop / t / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(rows)} of {M} rows of C (all {N} columns, K={K}), fp64 oracle, "
                      f"OpenMP over rows, {t:.1f} s",
            "single_thread": {"value": round(2.0 * n1 * N * K / t1 / 1e9, 3),
                              "unit": "GFLOP/s", "cores": 1,
                              "sample": f"{n1} of those rows on one thread, {t1:.2f} s"},
            "check_max_err": rep["max_err"], "check_nonfinite": rep["n_nonfinite"]}


def launch_stats(step, torch, dev, stream, steps: int, flush=None) -> dict:
    """Per-launch times from an event pair around each step (a separate pass after the
    timed region). With `flush`, a 512 MiB buffer is overwritten before each launch, outside
    its events, so every launch starts with A, B and C evicted from L2 and the memory-side
    cache (cold), instead of back to back (warm)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    n = len(ms)
    pick = lambda q: ms[min(n - 1, max(0, int(round(q * (n - 1)))))]
    return {"launches": n, "median_ms": round(pick(0.5), 5), "min_ms": round(ms[0], 5),
            "p90_ms": round(pick(0.9), 5), "mean_ms": round(sum(ms) / n, 5),
            "max_ms": round(ms[-1], 5)}


# Shapes of the plan check: one tile per CU and a few, ragged and square, short and deep
# K, low K with whole tiles, and large products.
PLAN_SWEEP_SHAPES = [
    (1024, 1024, 1024), (1024, 1024, 512), (1024, 1024, 2048), (1024, 1024, 4096),
    (1000, 1000, 1000), (1023, 1025, 1027), (768, 1024, 1024), (512, 512, 4096),
    (1024, 512, 2048), (1100, 1100, 1100), (1500, 1500, 1500), (2048, 2048, 2048),
    (2048, 2049, 2048), (2500, 2500, 2500), (3000, 3000, 3000), (1279, 1279, 2000),
    (2000, 2000, 1000), (1536, 1536, 1024), (1100, 1100, 4096), (900, 1300, 2500),
    (1200, 1200, 500), (5000, 5000, 1000), (4096, 4096, 4096), (4096, 4097, 4096),
    (6000, 6000, 6000), (8192, 8192, 1024), (4500, 4500, 8192), (3000, 3000, 8192),
    (16384, 16384, 64), (16384, 16384, 256), (4096, 4096, 256), (8192, 8192, 128),
    (256, 256, 32768), (512, 512, 8192), (2048, 2048, 8192), (700, 1300, 1500),
    (1000, 1000, 4000), (2000, 2000, 512), (1536, 3072, 1024), (3072, 3072, 2048)]


class SteadyTimer:
    """Times calls at steady state on cuda:0: at least 50 ms of a reference load first
    (2048^3 through sgemm_f32, on operands of its own), then each candidate runs for about
    1 ms of launches back to back (at least 5), in two passes (the second in reverse
    order), each after the same 5 ms of load; the faster pass counts. Over a pass the card
    warms and later candidates run at a lower clock, and the clock after a kernel depends
    on that kernel's power draw for some milliseconds: the reverse pass and the equal
    load before each candidate keep both from favouring a position."""

    H = 2048

    def __init__(self):
        import torch

        import fp32_gemm_f32_amd as g
        self.torch = torch
        self.lib = g.library()
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(self.dev)
        self.sp = self.stream.cuda_stream
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(17)
        H = self.H
        self.heat_ab = torch.randn((H, H), device=self.dev, generator=self.gen)
        self.heat_c = torch.empty((H, H), device=self.dev)
        self.timed(self.heat, 600)

    def heat(self):
        H = self.H
        assert self.heat_ab.numel() == H * H and self.heat_c.numel() == H * H
        return self.lib.sgemm_f32(H, H, H, self.heat_ab.data_ptr(), H, self.heat_ab.data_ptr(),
                                  H, self.heat_c.data_ptr(), H, self.sp)

    def timed(self, call, n):
        torch = self.torch
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(n):
            call()
        end.record(self.stream)
        torch.cuda.synchronize(self.dev)
        return start.elapsed_time(end) * 1e3 / n

    def operands(self, M, N, K):
        """Seeded normal A (M x K) and B (K x N) made on the device, and C (M x N)."""
        torch = self.torch
        A = torch.randn((M, K), device=self.dev, generator=self.gen)
        B = torch.randn((K, N), device=self.dev, generator=self.gen)
        return A, B, torch.empty((M, N), device=self.dev)

    def times(self, calls, n):
        """{name: microseconds per call} (None for a call that returns an error)."""
        times = {}
        for rnd in range(2):
            items = list(calls.items())
            for name, call in (items if rnd == 0 else items[::-1]):
                self.timed(self.heat, 40)
                if call() != 0:
                    times[name] = None
                    continue
                for _ in range(max(1, n // 4)):
                    call()
                t = self.timed(call, n)
                times[name] = t if times.get(name) is None else min(times[name], t)
        return times


def _sweep_shapes(spec: str):
    return (PLAN_SWEEP_SHAPES if spec == "default"
            else [tuple(int(x) for x in t.split("x")) for t in spec.split(",")])


def plan_sweep(spec: str, extra: str = "") -> int:
    """The plan's choice against every planned variant forced (and the variants named in
    `extra`, comma-separated, or every variant for 'all'), per shape, at steady state
    (SteadyTimer). The regret is the plan's variant's time over the fastest one's; the call
    through sgemm_f32 (the same kernel) is timed last in the first pass and reported
    beside. One JSON line per shape, then a summary line."""
    import fp32_gemm_f32_amd as g
    st = SteadyTimer()
    lib, sp = st.lib, st.sp
    names = g.variant_names()
    cands = g.planned_variants()
    if extra == "all":
        cands = list(range(len(names)))
    elif extra:
        cands += [names.index(x) for x in extra.split(",") if names.index(x) not in cands]
    regrets = []
    for (M, N, K) in _sweep_shapes(spec):
        A, B, C = st.operands(M, N, K)
        n = max(5, min(400, int(3e12 / (2.0 * M * N * K))))

        def gemm(v, A=A, B=B, C=C, M=M, N=N, K=K):
            # each call carries its own operands; their sizes are checked on the host
            assert A.shape == (M, K) and B.shape == (K, N) and C.shape == (M, N)
            if v < 0:
                return lib.sgemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(),
                                     N, sp)
            return lib.sgemm_f32_variant(v, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                         C.data_ptr(), N, sp)

        calls = {names[v]: (lambda v=v: gemm(v)) for v in cands}
        calls["auto"] = lambda: gemm(-1)
        times = st.times(calls, n)
        # the regret of the plan: its variant (forced, timed like the others) against the
        # fastest; the call through sgemm_f32 runs the same kernel and is reported beside
        plan = g.sgemm_f32_plan_describe(M, N, K)["name"]
        best = min((t, name) for name, t in times.items() if name != "auto" and t is not None)
        regret = times[plan] / best[0] - 1.0
        regrets.append(regret)
        print(json.dumps({"shape": [M, N, K], "plan": plan, "plan_us": round(times[plan], 2),
                          "auto_us": round(times["auto"], 2),
                          "best": best[1], "best_us": round(best[0], 2),
                          "regret": round(regret, 4),
                          "times_us": {k: (round(t, 2) if t is not None else None)
                                       for k, t in times.items()}}), flush=True)
    srt = sorted(regrets)
    print(json.dumps({"plan_sweep": {"shapes": len(srt), "max_regret": round(srt[-1], 4),
                                     "median_regret": round(srt[len(srt) // 2], 4),
                                     "within_1pct": sum(r <= 0.01 for r in srt)}}), flush=True)
    return 0


SPLIT_SWEEP_SHAPES = [
    (256, 256, 32768), (512, 512, 8192), (256, 256, 8192), (128, 128, 65536),
    (1024, 256, 16384), (512, 512, 32768), (384, 384, 16384), (640, 640, 8192),
    (2048, 256, 8192), (1024, 1024, 8192)]


def split_sweep(spec: str, splits: str) -> int:
    """Split-K's automatic split count (sgemm_f32_splitk with splits = 0) against the
    counts listed in `splits`, the plain plan (sgemm_f32) and stream-K's automatic choice,
    per shape, at steady state (SteadyTimer); each call includes its reduce or fixup
    kernel. The regret is the automatic count's time over the fastest split count's
    (1 being the plain plan). One JSON line per shape, then a summary line."""
    import fp32_gemm_f32_amd as g
    st = SteadyTimer()
    lib, sp, torch = st.lib, st.sp, st.torch
    counts = [int(x) for x in splits.split(",")]
    shapes = SPLIT_SWEEP_SHAPES if spec == "default" else _sweep_shapes(spec)
    regrets = []
    for (M, N, K) in shapes:
        A, B, C = st.operands(M, N, K)
        auto = lib.sgemm_f32_splitk_workspace_size(M, N, K, 0) // (4 * M * N) or 1
        need = max([lib.sgemm_f32_splitk_workspace_size(M, N, K, s) for s in counts + [auto]])
        ws = torch.empty(max(need // 4, 1), device=st.dev)
        sk_bytes = lib.sgemm_f32_streamk_workspace_size(M, N, K, K, N, N, -1)
        sw = torch.empty(max(sk_bytes // 4, 1), device=st.dev)
        n = max(5, min(400, int(3e12 / (2.0 * M * N * K))))

        def split(s, A=A, B=B, C=C, M=M, N=N, K=K, ws=ws):
            assert A.shape == (M, K) and B.shape == (K, N) and C.shape == (M, N)
            return lib.sgemm_f32_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(),
                                        N, s, ws.data_ptr(), ws.numel() * 4, sp)

        def streamk(A=A, B=B, C=C, M=M, N=N, K=K, sw=sw):
            assert A.shape == (M, K) and B.shape == (K, N) and C.shape == (M, N)
            return lib.sgemm_f32_streamk(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                         C.data_ptr(), N, -1, sw.data_ptr(), sw.numel() * 4, sp)

        calls = {"plain": lambda: split(1)}
        calls.update({f"splitk{s}": (lambda s=s: split(s)) for s in counts if s > 1})
        calls["splitk_auto"] = lambda: split(0)
        calls["streamk_auto"] = streamk
        times = st.times(calls, n)
        split_times = {k: t for k, t in times.items()
                       if k not in ("splitk_auto", "streamk_auto") and t is not None}
        best = min((t, k) for k, t in split_times.items())
        regret = times["splitk_auto"] / best[0] - 1.0
        regrets.append(regret)
        print(json.dumps({"shape": [M, N, K], "auto_splits": auto,
                          "auto_us": round(times["splitk_auto"], 2), "best": best[1],
                          "best_us": round(best[0], 2), "regret": round(regret, 4),
                          "times_us": {k: (round(t, 2) if t is not None else None)
                                       for k, t in times.items()}}), flush=True)
    srt = sorted(regrets)
    print(json.dumps({"split_sweep": {"shapes": len(srt), "max_regret": round(srt[-1], 4),
                                      "median_regret": round(srt[len(srt) // 2], 4),
                                      "within_2pct": sum(r <= 0.02 for r in srt)}}), flush=True)
    return 0


def bench_transpose(args) -> int:
    """The LDS bank-geometry microbenchmark: out = A^T for the workload's A (M x K)."""
    import torch

    import fp32_gemm_f32_amd as g
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    rows, cols = w.M, w.K
    tile, pad = int(args.kernel[9:11]), int(args.kernel[-1])
    A, _ = wl.operands(args.workload)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A).to(dev)
    dT = torch.empty((cols, rows), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = g.library()
    call = (rows, cols, dA.data_ptr(), cols, dT.data_ptr(), rows, tile, pad, stream.cuda_stream)
    for _ in range(args.warmup):
        lib.sgemm_f32_lds_transpose(*call)
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        rc = lib.sgemm_f32_lds_transpose(*call)
        if rc:
            raise g.SgemmError(rc, "sgemm_f32_lds_transpose")
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(end) / args.steps
    nbytes = 2.0 * 4 * rows * cols
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"bench: transpose {rows}x{cols} tile {tile} pad {pad}: {ms:.4f} ms, {gbs:.1f} GB/s")
    print(json.dumps({
        "metric": "LDS transpose GB/s (read + write)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"transpose of the {rows}x{cols} A operand of {w.name}",
                   "tile": tile, "pad": pad},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": None}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c3", "c4", "c5", "sk", "rk"])
    ap.add_argument("--variant", type=int, default=-1, help="force a hot-kernel tile variant")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "splitk", "streamk", "naive", "tiled16", "tiled32", "tiled32p", "regtiled41",
                             "regtiled44", "regtiled88", "transpose32p0", "transpose32p1",
                             "transpose64p0", "transpose64p1"],
                    help="the entry point a step calls (default: the hot path sgemm_f32); the "
                         "transposes move an M x N matrix of the workload's A shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time launches with L2 and the memory-side cache flushed before "
                         "each (512 MiB written between launches, outside the timed launch)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--plan-sweep", default="",
                    help="time the plan's choice against every planned variant at steady "
                         "state on 'default' (40 shapes) or a list MxNxK,MxNxK,...")
    ap.add_argument("--splits", type=int, default=0,
                    help="with --kernel splitk: the split count (0: the library's choice)")
    ap.add_argument("--split-sweep", default="",
                    help="time split-K's automatic split count against --sweep-splits, the "
                         "plain plan and stream-K on 'default' (10 under-filled shapes) or a "
                         "list MxNxK,...")
    ap.add_argument("--sweep-splits", default="2,4,8,16,32",
                    help="with --split-sweep: the split counts to time")
    ap.add_argument("--sweep-variants", default="",
                    help="with --plan-sweep: also time these variants (names, comma-separated; "
                         "'all' for every variant)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain device copy of this size instead (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py: runs on one GPU only; more than one GPU is not supported (a multi-GPU "
            "product would shard C by output tiles, each GPU running this kernel on its share)")
        return 2
    if args.plan_sweep:
        return plan_sweep(args.plan_sweep, args.sweep_variants)
    if args.split_sweep:
        return split_sweep(args.split_sweep, args.sweep_splits)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, max(args.steps, 1))
        return 0
    if args.kernel.startswith("transpose"):
        return bench_transpose(args)

    import torch

    import fp32_gemm_f32_amd as g
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    M, N, K = w.M, w.N, w.K
    log(f"bench: workload {w.describe()}, steps {args.steps}, warmup {args.warmup}")
    A, B = wl.operands(args.workload)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.empty((M, N), dtype=torch.float32, device=dev)
    plan = g.sgemm_f32_plan_describe(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                                     dC.data_ptr(), N)
    if args.variant >= 0:
        plan["name"] = g.variant_names()[args.variant]
    log(f"bench: plan {plan}")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    lib = g.library()
    call_args = (M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, sp)

    kern = args.kernel
    gemm = call_args[:-1]
    ws = None
    if kern == "splitk":
        ws_bytes = lib.sgemm_f32_splitk_workspace_size(M, N, K, args.splits)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        plan["splitk_workspace_bytes"] = ws_bytes
        plan["splits"] = ws_bytes // (4 * M * N) if ws_bytes else 1
        plan["name"] = (f"splitk{plan['splits']}+reduce" if plan["splits"] > 1
                        else "splitk1 (the plain plan)")
        plan["BM"] = plan["BN"] = plan["BK"] = plan["grid"] = None   # chosen per split count
    if kern == "streamk":
        sk_plan = g.sgemm_f32_streamk_describe(M, N, K, args.variant)
        ws_bytes = lib.sgemm_f32_streamk_workspace_size(M, N, K, K, N, N, args.variant)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        plan["streamk_workspace_bytes"] = ws_bytes
        plan["streamk_plan"] = sk_plan
        plan["name"] = (f"streamk_{sk_plan['name']}" if sk_plan["streamk"] else sk_plan["name"])
        plan["BM"], plan["BN"], plan["BK"] = sk_plan["BM"], sk_plan["BN"], sk_plan["BK"]
        plan["grid"] = (sk_plan["tiles_dp"] + sk_plan["G"] if sk_plan["streamk"]
                        else sk_plan["tiles"])
        log(f"bench: stream-K plan {sk_plan}")
    if kern not in ("auto", "splitk", "streamk"):
        plan["name"] = {"naive": "naive", "tiled16": "lds_tiled_16", "tiled32": "lds_tiled_32",
                        "tiled32p": "lds_tiled_32_padded", "regtiled41": "regtiled_4x1",
                        "regtiled44": "regtiled_4x4", "regtiled88": "regtiled_8x8"}[kern]
        plan["BM"] = plan["BN"] = plan["BK"] = plan["grid"] = None

    def step():
        if kern == "auto":
            rc = (lib.sgemm_f32(*call_args) if args.variant < 0
                  else lib.sgemm_f32_variant(args.variant, *call_args))
        elif kern == "splitk":
            rc = lib.sgemm_f32_splitk(*gemm, plan["splits"], ws.data_ptr(),
                                      plan["splitk_workspace_bytes"], sp)
        elif kern == "streamk":
            rc = lib.sgemm_f32_streamk(*gemm, args.variant, ws.data_ptr(),
                                       plan["streamk_workspace_bytes"], sp)
        elif kern == "naive":
            rc = lib.sgemm_f32_naive(*call_args)
        elif kern.startswith("tiled"):
            rc = lib.sgemm_f32_tiled(*gemm, int(kern[5:7]), 1 if kern.endswith("p") else 0, sp)
        else:
            rc = lib.sgemm_f32_regtiled(*gemm, int(kern[8]), int(kern[9]), sp)
        if rc != 0:
            raise g.SgemmError(rc, kern)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t_wall0
    elapsed_ms = start.elapsed_time(end)
    ms = elapsed_ms / args.steps
    flop = 2.0 * M * N * K
    gflops = flop * args.steps / (elapsed_ms / 1e3) / 1e9
    log(f"bench: {ms:.4f} ms/step (events), wall {wall:.3f} s, {gflops:.1f} GFLOP/s")

    # per-launch statistics, in passes of their own after the timed region
    timing = {"region_ms_per_step": round(ms, 5),
              "host_us_per_call": round(wall / args.steps * 1e6, 2),
              "warm": launch_stats(step, torch, dev, stream, args.steps)}
    if args.cold:
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        timing["cold"] = launch_stats(step, torch, dev, stream, args.steps, flush)
        del flush
    log(f"bench: per-launch timing {timing}")

    # roofline of the one kernel a step launches
    compulsory = 4.0 * (M * K + K * N + M * N)
    t_mfma = flop / (PEAK_FP32_MFMA_TFLOPS * 1e12)
    t_hbm = compulsory / (PEAK_HBM_GBS * 1e9)
    t_step = ms / 1e3
    if kern not in ("auto", "splitk", "streamk"):
        # the scalar rungs run on the vector ALUs without packed FP32: 256 CUs x 4 SIMDs x
        # 16 lanes x 2 FLOP x 2.4 GHz
        achieved = flop / (ms / 1e3) / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_FP32_VALU_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_VALU_TFLOPS, 4)}
    elif t_mfma >= t_hbm:
        achieved = flop / (ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4)}
    else:
        achieved = compulsory / (ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = (measured_traffic(args.workload, plan["name"])
                       if kern == "auto" and args.variant < 0 else None)
    roof["kernel"] = plan["name"]
    # both floors against the measured step, whichever binds: the FP32 matrix floor 2MNK /
    # 157.3 TFLOP/s and the HBM floor 4 (MK + KN + MN) / 8 TB/s (read A and B, write C once)
    roof["frac_mfma"] = round(t_mfma / t_step, 4)
    roof["frac_hbm"] = round(t_hbm / t_step, 4)
    roof["compulsory_bytes"] = int(compulsory)
    if roof["traffic"]:
        roof["traffic_over_compulsory"] = round(roof["traffic"] / compulsory, 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A, B, dC, M, N, K, args.cpu_seconds)
        log(f"bench: cpu baseline {cpu}")
        if cpu["check_nonfinite"] or cpu["check_max_err"] > 1e-5:
            log("bench: PARITY FAILURE on the sampled rows")
            return 1

    out = {
        "metric": "SGEMM GFLOP/s (2MNK/t) and % of FP32 matrix peak at 8192^3, 1 MI355X",
        "value": round(gflops, 1), "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": f"{w.label} ({w.name}): FP32 row-major C=AxB, "
                               f"{w.dist} operands from fixed seeds",
                   "M": M, "N": N, "K": K, "lda": K, "ldb": N, "ldc": N,
                   "kernel": plan["name"], "tile": [plan["BM"], plan["BN"], plan["BK"]],
                   "grid": plan["grid"], "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing": timing,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
