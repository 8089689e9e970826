"""Build the HIP library libsgemm_f32.so in-tree for gfx950 with hipcc.

    python -m fp32_gemm_f32_amd.build           # build
    python -m fp32_gemm_f32_amd.build --asm     # also write the gfx950 assembly

The resource usage of every kernel (VGPRs, AGPRs, LDS, occupancy) is written to
fp32_gemm_f32_amd/_build/resource_usage.txt from the compiler's own report.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libsgemm_f32.so")
BUILD_DIR = os.path.join(PKG, "_build")
# Translation units and whether their MFMA accumulators are held in VGPRs (see flags()).
# The one-wave-per-SIMD kernel keeps 256 accumulators per lane in AGPRs, so it is compiled
# on its own, without that option.
SOURCES = [(os.path.join(CSRC, "sgemm_f32.hip"), True),
           (os.path.join(CSRC, "sgemm_regpanel.hip"), False),
           (os.path.join(CSRC, "sgemm_persist.hip"), False)]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags(vgpr_form: bool = True) -> list[str]:
    f = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed FP32 instructions stay off: the compiler must not form them from float2
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]
    if vgpr_form:
        # MFMA accumulators stay in VGPRs (every kernel of the unit fits in 256 registers);
        # left to its heuristics the register allocator moves them between AGPRs and VGPRs
        # on each iteration of the persistent stream-K tile loop
        f += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return f


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    report = os.path.join(BUILD_DIR, "resource_usage.txt")
    objs, log = [], []
    for src, vgpr_form in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *flags(vgpr_form), "-c", src, "-o", obj,
               "-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        log.append(r.stderr)
        if r.returncode != 0:
            with open(report, "w") as f:
                f.write("".join(log))
            sys.stderr.write(r.stderr[-8000:])
            raise RuntimeError(f"hipcc failed ({r.returncode}) on {src}; see {report}")
        objs.append(obj)
    with open(report, "w") as f:
        f.write("".join(log))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr[-8000:])
        raise RuntimeError(f"hipcc link failed ({r.returncode})")
    check_symbols(OUT + ".tmp")
    os.replace(OUT + ".tmp", OUT)
    if asm:
        assemble()
    return OUT


def check_symbols(lib: str) -> None:
    """Fail on any undefined symbol of the library's own namespace. The compiler can drop a
    kernel template's host stub without a diagnostic (and exit 0); the library then fails
    to load only where it is used, so the build refuses it here."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}: {r.stderr[-2000:]}")
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN5sgemm" in l]
    if missing:
        raise RuntimeError("library has undefined kernel symbols (host stubs not emitted): " +
                           ", ".join(missing[:8]))


def assemble(out: str | None = None) -> str:
    """Write the gfx950 assembly of the library's device code (same flags as the build),
    all translation units into one file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    s = out or os.path.join(BUILD_DIR, "sgemm_f32.s")
    parts = []
    for src, vgpr_form in SOURCES:
        part = s + "." + os.path.basename(src) + ".s"
        subprocess.run([hipcc(), *flags(vgpr_form), "--cuda-device-only", "-S", src, "-o", part],
                       check=True)
        with open(part) as f:
            parts.append(f.read())
        os.remove(part)
    with open(s, "w") as f:
        f.write("\n".join(parts))
    return s


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, verbose=a.verbose))


if __name__ == "__main__":
    main()
