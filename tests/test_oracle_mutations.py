"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins
catch every one: a pin suite that passes a broken oracle would not be a pin.

Each mutant is built from the oracle's C source by one textual substitution and run in
a child process (a mutant may read out of bounds), which reports the pins that failed.
"""
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sgemm_oracle.c")

# (name, original text, mutated text, occurrence to replace: 0 = first, 1 = second, ...)
MUTANTS = [
    ("dropped_last_term", "for (int64_t k = 0; k < K; ++k) {\n            const double a",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a", 0),
    ("skipped_first_term", "for (int64_t k = 0; k < K; ++k) {\n            const double a",
     "for (int64_t k = 1; k < K; ++k) {\n            const double a", 0),
    ("wrong_sign", "c[j] += a * (double)b[j];", "c[j] -= a * (double)b[j];", 0),
    ("transposed_A", "const double a = (double)A[i * lda + k];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]",
     "const double a = (double)A[k * lda + i];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]", 0),
    ("B_row_uses_i", "const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]",
     "const float *b = B + (k + i) % K * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]", 0),
    ("A_stride_ldb", "const double a = (double)A[i * lda + k];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]",
     "const double a = (double)A[i * ldb + k];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j]", 0),
    ("float_accumulate", "double *c = C + i * ldc;\n        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;\n        for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[j];",
     "double *c = C + i * ldc;\n        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;\n        for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float *b = B + k * ldb;\n            for (int64_t j = 0; j < N; ++j) c[j] = (float)(c[j] + (float)(a * (double)b[j]));", 0),
    ("row_den_signed", "den[j] += fabs(p);", "den[j] += p;", 0),
    ("row_dropped_last_term", "for (int64_t k = 0; k < K; ++k) {\n        const double a = (double)A[i * lda + k];\n        const float *b = B + k * ldb;\n        for (int64_t j = 0; j < N; ++j) {",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n        const double a = (double)A[i * lda + k];\n        const float *b = B + k * ldb;\n        for (int64_t j = 0; j < N; ++j) {", 0),
    ("check_inexact_never", "if (c != (float)acc[j]) mine.n_inexact++;", "if (c != c) mine.n_inexact++;", 0),
    ("check_err_unnormalised", "err = fabs((double)c - acc[j]) / den[j];", "err = fabs((double)c - acc[j]);", 0),
    ("check_nan_passes", "if (!isfinite(c)) {", "if (0) {", 0),
    ("sample_wrong_B_index", "(double)B[k * ldb + jj[t]]", "(double)B[jj[t] * ldb + k]", 0),
    ("sample_den_signed", "d += fabs(p);", "d += p;", 0),
    ("transpose_not_transposed", "out[j * ldo + i] = in[i * ldi + j];", "out[i * ldo + j] = in[i * ldi + j];", 0),
]

# Mutants of the routines behind oracle.check (oracle_row) and oracle.sample, which every
# GPU parity verdict rests on. Each names the pin that must catch it, and the pin run must
# end normally: a catch may not come from an out-of-bounds read crashing the run. The
# integer pins run square shapes first, where a transposed or mis-strided index still reads
# inside the operands.
_ROW_A = ("const double a = (double)A[i * lda + k];\n        const float *b = B + k * ldb;\n"
          "        for (int64_t j = 0; j < N; ++j) {")
_ROW_B = "const double p = a * (double)b[j];"
NAMED_MUTANTS = [
    ("row_A_column_fixed", _ROW_A, _ROW_A.replace("A[i * lda + k]", "A[i * lda]"),
     "pin_check_integer"),
    ("row_A_transposed", _ROW_A, _ROW_A.replace("A[i * lda + k]", "A[k * lda + i]"),
     "pin_check_integer"),
    ("row_A_stride_ldb", _ROW_A, _ROW_A.replace("A[i * lda + k]", "A[i * ldb + k]"),
     "pin_check_integer"),
    ("row_A_row_fixed", _ROW_A, _ROW_A.replace("A[i * lda + k]", "A[k]"),
     "pin_check_integer"),
    ("row_B_column_from_i", _ROW_B, "const double p = a * (double)b[i % N];",
     "pin_check_integer"),
    ("row_B_row_from_i", _ROW_A, _ROW_A.replace("B + k * ldb", "B + (i % K) * ldb"),
     "pin_check_integer"),
    ("row_B_transposed", _ROW_B, "const double p = a * (double)B[j * ldb + k];",
     "pin_check_integer"),
    ("check_rows_ignored", "const int64_t i = rows ? rows[t] : t;",
     "const int64_t i = t;", "pin_check_integer"),
    ("check_arg_j_dropped", "mine.max_err = err; mine.arg_i = i; mine.arg_j = j;",
     "mine.max_err = err; mine.arg_i = i; mine.arg_j = 0;", "pin_check_integer"),
    ("sample_A_transposed", "(double)A[ii[t] * lda + k]", "(double)A[k * lda + ii[t]]",
     "pin_sample_integer"),
    ("sample_A_column_fixed", "(double)A[ii[t] * lda + k]", "(double)A[ii[t] * lda]",
     "pin_sample_integer"),
    ("sample_B_column_from_i", "(double)B[k * ldb + jj[t]]", "(double)B[k * ldb + ii[t] % N]",
     "pin_sample_integer"),
]


def _mutate(src: str, old: str, new: str, occurrence: int) -> str:
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old[:60]!r}"
    return src[:pos] + new + src[pos + len(old):]


RUNNER = r"""
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load({lib!r})
failed = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except AssertionError:
        failed.append(pin.__name__)
    except Exception as e:
        failed.append(pin.__name__ + ":" + type(e).__name__)
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ, tmp_path):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    csrc = tmp_path / f"{name}.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / f"{name}.so")
    oracle.build(str(csrc), lib)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, env=dict(os.environ, OMP_NUM_THREADS="2"))
    if r.returncode != 0:
        return  # the mutant crashed the pin run: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"


def _run_pins(name, old, new, tmp_path):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, 0)
    assert mutated != src
    csrc = tmp_path / f"{name}.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / f"{name}.so")
    oracle.build(str(csrc), lib)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, env=dict(os.environ, OMP_NUM_THREADS="2"))


@pytest.mark.parametrize("name,old,new,pin", NAMED_MUTANTS, ids=[m[0] for m in NAMED_MUTANTS])
def test_named_mutant_is_caught(name, old, new, pin, tmp_path):
    r = _run_pins(name, old, new, tmp_path)
    assert r.returncode == 0, f"mutant {name} crashed the pin run: {r.stderr[-400:]}"
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert pin in failed, f"mutant {name} passed {pin} (failed: {failed})"
