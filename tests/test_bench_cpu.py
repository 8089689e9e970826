"""Host-side pieces of bench.py: the multi-GPU refusal and the machine-code hash that decides
whether the committed HBM counters still apply."""
import json
import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_code_hash(tmp_path):
    """Every kernel of the built library gets a hash of its own gfx950 machine code; the
    hashes are stable, differ between kernels, and are None for a file that is not such a
    library or a kernel that is not in it."""
    syms = bench.kernel_symbols()
    mfma = [s for s in syms if "k_sgemm_mfma" in s]
    assert len(mfma) >= 5 and any("k_splitk_reduce" in s for s in syms)
    assert all(len(h) == 16 for h in syms.values())
    assert len(set(syms[s] for s in mfma)) == len(mfma)
    assert bench.kernel_code_hash(mfma[0]) == syms[mfma[0]] == bench.kernel_symbols()[mfma[0]]
    assert bench.kernel_code_hash("no_such_kernel") is None
    junk = tmp_path / "not_a_library.so"
    junk.write_bytes(b"not an ELF file at all" * 10)
    assert bench.kernel_symbols(str(junk)) == {}
    # the library holds one offload bundle per translation unit; kernels of both are found
    assert any("k_sgemm_regpanel" in s for s in syms)
    assert bench.kernel_code_hash(mfma[0], str(tmp_path / "missing.so")) is None


def test_traffic_needs_matching_variant():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    for name, entry in data.items():
        if not name.startswith("_"):
            assert bench.measured_traffic(name, entry["variant"] + "_other") is None


def test_committed_traffic_entries_are_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    cal = data["_calibration"]
    assert 1.5 < cal["fetch_scale"] < 2.5 and 0.8 < cal["write_scale"] < 1.2
    for name, entry in data.items():
        if name.startswith("_"):
            continue
        assert entry["bytes_per_launch"] >= entry["compulsory_bytes"] * 0.9, name
        # a tile variant's name, or a stream-K plan's ("streamk_" + the variant's)
        variant = entry["variant"].removeprefix("streamk_")
        assert len(entry["kernel_code_sha"]) == 16 and variant.startswith("mfma")
        assert entry["kernel_symbol"].startswith(("_ZN5sgemm12k_sgemm_mfma",
                                                  "_ZN5sgemm16k_sgemm_regpanel",
                                                  "_ZN5sgemm15k_sgemm_persist"))


def test_default_workload_traffic_is_current():
    """The default bench line (8192^3) reports measured HBM traffic only while the counters
    were taken on the machine code that runs now: the committed record must match the
    current build's kernel and plan."""
    import fp32_gemm_f32_amd as g
    plan = g.sgemm_f32_plan_describe(8192, 8192, 8192, 1 << 40, None, (1 << 40) + (1 << 30),
                                     None, (1 << 40) + (1 << 31), None, num_cus=256)
    assert bench.measured_traffic("c4", plan["name"]) is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
