"""Every plausible slip in the oracle must fail at least one pin.

Each mutant is a copy of the oracle's C source with one deliberate mistake
(planted here, on the CPU, in a temporary copy; the real oracle is never
touched).  The copy is compiled with the same flags and the whole pin suite
runs against it in a child process, so a mutant that crashes is contained.
A mutant that passes every pin would mean the pins leave that part of the
oracle unchecked.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as obuild  # noqa: E402

# (name, text in the source, replacement)
MUTANTS = [
    ("drop_last_k", "for (long k = 0; k < K; ++k) {", "for (long k = 0; k < K - 1; ++k) {"),
    ("skip_first_k", "for (long k = 0; k < K; ++k) {", "for (long k = 1; k < K; ++k) {"),
    ("transposed_B", "S[j] += a * (double)Bk[j];", "S[j] += a * (double)B[j * ldb + k];"),
    ("ignore_lda", "const double a = (double)A[i * lda + k];", "const double a = (double)A[i * K + k];"),
    ("ignore_ldb", "const float *Bk = B + k * ldb;", "const float *Bk = B + k * N;"),
    ("ignore_ldc", "const float *c = C_in + i * ldc;", "const float *c = C_in + i * N;"),
    ("beta_sign", "o[j] = a_s * S[j] + b_s * (double)c[j];", "o[j] = a_s * S[j] - b_s * (double)c[j];"),
    ("alpha_dropped_beta0", "for (long j = 0; j < N; ++j) o[j] = a_s * S[j];",
     "for (long j = 0; j < N; ++j) o[j] = S[j];"),
    ("alpha_dropped_beta", "o[j] = a_s * S[j] + b_s * (double)c[j];", "o[j] = S[j] + b_s * (double)c[j];"),
    ("reads_c_when_beta0", "if (beta == 0.0f) {", "if (beta == 0.0f && C_in == NULL) {"),
    ("float_accumulator", "S[j] += a * (double)Bk[j];", "S[j] = (float)(S[j] + a * (double)Bk[j]);"),
    ("float_epilogue", "for (long j = 0; j < N; ++j) o[j] = a_s * S[j];",
     "for (long j = 0; j < N; ++j) o[j] = (float)(a_s * S[j]);"),
    ("swapped_a_index", "const double a = (double)A[i * lda + k];",
     "const double a = (double)A[(k % M) * lda + (i % K)];"),
    ("stale_row_accumulator", "for (long j = 0; j < N; ++j) S[j] = 0.0;", ";"),
    ("sampled_drops_beta", "if (beta != 0.0f) v = v + b_s * (double)C_in[i * ldc + j];", ";"),
    ("sampled_wrong_column", "S += (double)A[i * lda + k] * (double)B[k * ldb + j];",
     "S += (double)A[i * lda + k] * (double)B[k * ldb + (j + 1) % N];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = src.replace(old, new)
    csrc = tmp_path / f"oracle_{name}.c"
    lib = tmp_path / f"liboracle_{name}.so"
    csrc.write_text(mutated)
    subprocess.run(["gcc", *obuild.CFLAGS, str(csrc), "-o", str(lib)], check=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), "--lib", str(lib)],
                       capture_output=True, text=True, timeout=600,
                       env={**os.environ, "OMP_NUM_THREADS": "4"})
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"
