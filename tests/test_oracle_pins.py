"""The CPU oracle against its pins (closed forms, invariants, exact brute force)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_thread_count_invariance(lib, monkeypatch):
    """Rows are independent: a 1-thread run gives the same bits as the default run."""
    import subprocess, sys, os, json
    code = (
        "import numpy as np, oracle, json;"
        "rng=np.random.default_rng(5);"
        "A=rng.uniform(-1,1,(67,301)).astype(np.float32);"
        "B=rng.uniform(-1,1,(301,45)).astype(np.float32);"
        "print(json.dumps(oracle.gemm_f64(A,B).ravel().tolist()))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for threads in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=threads, PYTHONPATH=root)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, check=True)
        outs.append(json.loads(r.stdout))
    assert outs[0] == outs[1]
