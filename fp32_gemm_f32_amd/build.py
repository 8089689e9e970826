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
SOURCES = [os.path.join(CSRC, "sgemm_f32.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed FP32 instructions stay off: the compiler must not form them from float2
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators stay in VGPRs (every kernel fits in 256 registers); left to its
        # heuristics the register allocator moves them between AGPRs and VGPRs on each
        # iteration of the persistent tile loop
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    report = os.path.join(BUILD_DIR, "resource_usage.txt")
    cmd = [hipcc(), *flags(), "-shared", *SOURCES, "-o", OUT + ".tmp",
           "-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    with open(report, "w") as f:
        f.write(r.stderr)
    if r.returncode != 0:
        sys.stderr.write(r.stderr[-8000:])
        raise RuntimeError(f"hipcc failed ({r.returncode}); see {report}")
    os.replace(OUT + ".tmp", OUT)
    if asm:
        assemble()
    return OUT


def assemble(out: str | None = None) -> str:
    """Write the gfx950 assembly of the library's device code (same flags as the build)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    s = out or os.path.join(BUILD_DIR, "sgemm_f32.s")
    subprocess.run([hipcc(), *flags(), "--cuda-device-only", "-S", *SOURCES, "-o", s],
                   check=True)
    return s


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, verbose=a.verbose))


if __name__ == "__main__":
    main()
