"""Machine-code check of the built gfx950 kernels: store-data wait states.

A vector store wider than 64 bits reads its data registers after it issues, and on gfx950
a VALU write to those registers right behind it corrupts lanes of the stored data. The
compiler's hazard model leaves out stores whose soffset is an SGPR, so the kernels must
keep the gap themselves. This scans the gfx950 assembly of the library for a VALU
instruction writing a data register of such a store with fewer than `need` wait states
in between (s_nop N gives N + 1, any other instruction 1).

    python -m fp32_gemm_f32_amd.asm_check     # builds the assembly, exits 1 on a finding
"""
from __future__ import annotations

import re
import sys

WIDE_STORES = ("buffer_store_dwordx4", "buffer_store_dwordx3", "global_store_dwordx4",
               "global_store_dwordx3", "flat_store_dwordx4", "flat_store_dwordx3")
# instructions that write no VGPR (their first operand is an SGPR or VCC)
NO_VGPR_WRITE = ("v_readlane", "v_readfirstlane", "v_cmp")


def _vgprs(tok: str) -> set[int]:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _data_operand(op: str) -> int:
    """Position of the data registers among a store's operands: first for buffer stores
    (vdata, vaddr, srsrc, soffset), second for global and flat stores (vaddr, vdata, ...)."""
    return 1 if op.startswith("buffer_") else 2


def store_data_hazards(asm: str, need: int = 2) -> dict[str, list[tuple[int, str, str]]]:
    """Kernel symbol -> [(wait states, store, writing instruction)] for every finding."""
    kernel, insts, hits = None, [], {}
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kernel, insts = m.group(1), []
            continue
        s = line.strip()
        if kernel is None or not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        op = s.split()[0]
        if op.startswith("v_") and not op.startswith(NO_VGPR_WRITE) and len(s.split()) > 1:
            written = _vgprs(s.split()[1].rstrip(","))
            waits = 0
            for prev in reversed(insts[-8:]):
                if waits >= need:
                    break
                p = prev.split()
                if p[0].startswith(WIDE_STORES) and written & _vgprs(p[_data_operand(p[0])].rstrip(",")):
                    hits.setdefault(kernel, []).append((waits, prev, s))
                    break
                waits += int(p[1]) + 1 if p[0] == "s_nop" else 1
        insts.append(s)
    return hits


def main() -> int:
    from fp32_gemm_f32_amd import build
    path = build.assemble()
    hits = store_data_hazards(open(path).read())
    for k, v in hits.items():
        print(f"{k}: {len(v)} stores, e.g. {v[0]}")
    print(f"{path}: {len(hits)} kernels with store-data hazards")
    return 1 if hits else 0


if __name__ == "__main__":
    sys.exit(main())
