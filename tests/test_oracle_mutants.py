"""The pins of tests/test_oracle.py catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake in the copy (a wrong
sign, a dropped term, a transposed operand, a wrong head or checkpoint index, a
wrong gate), builds it into a temporary library on the CPU and runs the pins
against it: at least one pin must fail.  The real oracle is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import tests.test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "update_sign": ("alpha * (S[i * dk + j] - beta * u[i] * kt[j])",
                    "alpha * (S[i * dk + j] + beta * u[i] * kt[j])"),
    "drop_write_term": ("+\n                          beta * vt[i] * kt[j];", ";"),
    "transposed_state_in_Sk": ("acc += S[i * dk + j] * kt[j];", "acc += S[j * dk + i] * kt[j];"),
    "output_uses_key": ("acc += S[i * dk + j] * qt[j];", "acc += S[i * dk + j] * kt[j];"),
    "beta_outside_decay": ("alpha * (S[i * dk + j] - beta * u[i] * kt[j])",
                           "alpha * S[i * dk + j] - beta * u[i] * kt[j]"),
    "head_interleaved": ("hq = h / group;\n    double *S = S_final + unit * unit_sz;",
                         "hq = h % Hqk;\n    double *S = S_final + unit * unit_sz;"),
    "checkpoint_off_by_one": ("const int slot = t - (L[r] - nt);", "const int slot = t - (L[r] - nt) - 1;"),
    "softplus_sign": ("log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    "sigmoid_sign": ("beta[i] = 1.0 / (1.0 + exp(-b[i]));", "beta[i] = 1.0 / (1.0 + exp(b[i]));"),
    "decay_rate_sign": ("return -exp(A_log) * softplus(a + dt_bias);",
                        "return -exp(-A_log) * softplus(a + dt_bias);"),
    "dt_bias_dropped": ("softplus(a + dt_bias)", "softplus(a)"),
    "chunk_U_sign": ("U[t * dv + i] = acc - ws;", "U[t * dv + i] = acc + ws;"),
    "chunk_gamma_reversed": ("const double coef = exp(G[t] - G[s]) * qk;",
                             "const double coef = exp(G[s] - G[t]) * qk;"),
}

# pins run against every mutant (square shapes only: a transposed index on a
# non-square state would read outside the copy's buffers)
PINS = [
    pins.test_gates_match_library_routines,
    pins.test_hand_worked_2x2_example,
    lambda: pins.test_brute_force_transition_matrices(1, 1, 16, 16, [12]),
    lambda: pins.test_brute_force_transition_matrices(2, 4, 16, 16, [5, 1, 9]),
    lambda: pins.test_chunked_form_equals_sequential(8, 0.0),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(src), "-lm"],
                   check=True)
    saved = oracle._lib
    oracle._lib = None
    try:
        real = oracle._LIB
        oracle._LIB = str(so)  # loader picks up the mutant (its mtime is newer than the source)
        oracle._load()
        caught = []
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin)
        assert caught, "no pin caught the planted mistake %r" % name
    finally:
        oracle._LIB = real
        oracle._lib = saved
