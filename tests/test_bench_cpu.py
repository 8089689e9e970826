"""Host-side pieces of bench.py: the JSON contract's fixed fields, the multi-GPU refusal and
the kernel-source hash that decides whether the committed HBM counters still apply."""
import json
import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_strip_comments_ignores_comments_and_layout():
    a = 'int f(int x) { // add one\n  return x + 1; /* done */ }\nconst char *s = "// not a comment";\n'
    b = 'int f(int x)\n{\n    return x + 1;\n}\n/* a new\n   block comment */\nconst char *s = "// not a comment";'
    assert bench.strip_comments(a).split() == bench.strip_comments(b).split()
    assert '"// not a comment"' in bench.strip_comments(a)
    c = a.replace("x + 1", "x + 2")
    assert bench.strip_comments(c) != bench.strip_comments(a)


def test_kernel_hash_is_stable_and_sized():
    h = bench.kernel_sources_hash()
    assert h == bench.kernel_sources_hash() and len(h) == 16


def test_committed_traffic_entries_are_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    cal = data["_calibration"]
    assert 1.5 < cal["fetch_scale"] < 2.5 and 0.8 < cal["write_scale"] < 1.2
    for name, entry in data.items():
        if name.startswith("_"):
            continue
        assert entry["bytes_per_launch"] >= entry["compulsory_bytes"] * 0.9, name
        assert len(entry["kernel_sources_sha"]) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
