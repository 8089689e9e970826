"""Host-side pieces of bench.py: the multi-GPU refusal and the machine-code hash that decides
whether the committed HBM counters still apply."""
import json
import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_code_hash(tmp_path):
    """The hash covers the gfx950 code object inside the built library, is stable, and is
    None for a file that is not such a library."""
    h = bench.kernel_code_hash()
    assert h is not None and len(h) == 16 and h == bench.kernel_code_hash()
    junk = tmp_path / "not_a_library.so"
    junk.write_bytes(b"not an ELF file at all" * 10)
    assert bench.kernel_code_hash(str(junk)) is None
    assert bench.kernel_code_hash(str(tmp_path / "missing.so")) is None


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
        assert len(entry["kernel_code_sha"]) == 16 and entry["variant"].startswith("mfma_")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
