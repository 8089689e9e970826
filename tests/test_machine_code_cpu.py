"""The gfx950 machine code keeps two wait states between every vector store wider than 64
bits and any VALU write of its data registers (a hazard the compiler does not model for
stores with an SGPR soffset; without the gap the stream-K kernels stored corrupted lanes).
Builds the assembly with the library's own flags; no GPU needed."""
import shutil

import pytest

from fp32_gemm_f32_amd import asm_check, build


def test_scanner_finds_the_pattern():
    bad = """_ZN5sgemm4kernE:
\tbuffer_store_dwordx4 v[2:5], v1, s[8:11], s3 offen nt
\tv_mov_b32_e32 v2, v17
"""
    ok_gap = bad.replace("\tv_mov_b32_e32 v2, v17", "\ts_nop 1\n\tv_mov_b32_e32 v2, v17")
    other_reg = bad.replace("v2, v17", "v6, v17")
    narrow = bad.replace("dwordx4 v[2:5]", "dwordx2 v[2:3]")
    assert list(asm_check.store_data_hazards(bad)) == ["_ZN5sgemm4kernE"]
    assert asm_check.store_data_hazards(ok_gap) == {}
    assert asm_check.store_data_hazards(other_reg) == {}
    assert asm_check.store_data_hazards(narrow) == {}
    one_gap = bad.replace("\tv_mov_b32_e32 v2, v17", "\ts_movk_i32 s4, 0x400\n\tv_mov_b32_e32 v2, v17")
    assert asm_check.store_data_hazards(one_gap)          # 1 wait state is not enough
    assert asm_check.store_data_hazards(one_gap, need=1) == {}
    # global stores name the address first and the data second
    glob = """_ZN5sgemm4kernE:
\tglobal_store_dwordx4 v[2:3], v[6:9], off offset:-8
\tv_lshl_add_u64 v[2:3], v[2:3], 0, 16
"""
    assert asm_check.store_data_hazards(glob) == {}
    assert list(asm_check.store_data_hazards(glob.replace("v[2:3], v[2:3], 0, 16",
                                                          "v[6:7], v[2:3], 0, 16"))) == \
        ["_ZN5sgemm4kernE"]


@pytest.mark.skipif(shutil.which("hipcc") is None and not build.os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_built_kernels_keep_store_data_gap(tmp_path):
    path = build.assemble(str(tmp_path / "sgemm_f32.s"))
    text = open(path).read()
    assert "k_sgemm_mfma" in text and "k_streamk_fixup" in text
    hits = asm_check.store_data_hazards(text)
    assert hits == {}, {k: v[:2] for k, v in hits.items()}
