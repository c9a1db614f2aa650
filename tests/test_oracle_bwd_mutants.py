"""The backward oracle's pins must catch plausible slips: each mutant is a copy of the
oracle source with one planted mistake in the gradient code, compiled on the CPU, and at
least one pin in test_oracle_bwd.py has to fail against it. Every mutant keeps all
memory accesses in bounds.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_bwd as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "softmax Jacobian without the row term (dQ)":
        ("double ds = p * (dprob(dout, v, dtype, Nq, Nk, d, r, j) - dsum);",
         "double ds = p * dprob(dout, v, dtype, Nq, Nk, d, r, j);"),
    "softmax Jacobian without the row term (dK)":
        ("double ds = p * (dprob(dout, v, dtype, Nq, Nk, d, r, j) - dsum_all[r]);",
         "double ds = p * dprob(dout, v, dtype, Nq, Nk, d, r, j);"),
    "dK without the scale": ("gk[t] += scale * ds * widen(q, dtype, off + t);",
                             "gk[t] += ds * widen(q, dtype, off + t);"),
    "dQ sums values instead of keys": ("out[t] += scale * ds * widen(k, dtype, koff + t);",
                                       "out[t] += scale * ds * widen(v, dtype, koff + t);"),
    "dV weighted by dS": ("gv[t] += p * widen(dout, dtype, off + t);",
                          "gv[t] += ds * widen(dout, dtype, off + t);"),
    "P not normalised": ("double p = exp(sc - lse_all[r]);", "double p = exp(sc);"),
    "dP from the query row": ("size_t ooff = (size_t)r * d, voff = ((size_t)bh * Nk + j) * d;",
                              "size_t ooff = (size_t)r * d, voff = (size_t)r * d;"),
    "causal mask ignored in the gradient":
        ("if (causal && (long long)j - query_offset(causal, Nq, Nk) > (long long)i) return -INFINITY;",
         "(void)i;"),
}

PINS = [
    lambda: pins.test_finite_differences(False, 5, 7),
    lambda: pins.test_finite_differences(True, 4, 9),
    lambda: pins.test_matches_torch_autograd_float64(True, 17, 50, 32),
    lambda: pins.test_invariants(True),
    pins.test_single_key_and_zero_upstream,
    pins.test_equal_value_rows_give_no_score_gradient,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_mutant(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name!r} not found exactly once"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(mut), "-o", lib_path, "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(lib_path))
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin caught the mutant {name!r}"


def test_unmutated_source_passes_every_bwd_pin():
    for pin in PINS:
        pin()
