"""The oracle's pins must catch plausible slips: each mutant below is a copy of the oracle
source with one planted mistake, compiled on the CPU, and at least one pin in
test_oracle.py has to fail against it. Every mutant keeps all memory accesses in bounds.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "no max subtraction": ("exp(s[j] - m)", "exp(s[j])"),
    "causal ignores the Nk-Nq offset": ("(long long)i + query_offset(causal, Nq, Nk)", "(long long)i"),
    "top-left alignment uses the bottom-right offset": ("return causal == 2 ? 0 : (long long)Nk - (long long)Nq;",
                                                       "return (long long)Nk - (long long)Nq;"),
    "top-left alignment shifted by one": ("return causal == 2 ? 0 : (long long)Nk - (long long)Nq;",
                                          "return causal == 2 ? 1 : (long long)Nk - (long long)Nq;"),
    "causal off by one": ("(long long)j > last_visible", "(long long)j >= last_visible"),
    "K operand transposed": ("widen(k, dtype, kvbase + (size_t)j * d + t)",
                             "widen(k, dtype, kvbase + (size_t)t * Nk + j)"),
    "V replaced by K": ("widen(v, dtype, kvbase + (size_t)j * d + t)",
                        "widen(k, dtype, kvbase + (size_t)j * d + t)"),
    "no normalisation": ("double w = s[j] / l;", "double w = s[j];"),
    "LSE sign": ("*lse = m + log(l);", "*lse = m - log(l);"),
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "empty row gets LSE 0": ("*lse = -INFINITY;", "*lse = 0.0;"),
    "bf16 widened from the wrong bits": ("<< 16;", "<< 15;"),
    "query row taken from head 0": ("size_t qoff = (size_t)r * (size_t)d;",
                                    "size_t qoff = (size_t)i * (size_t)d;"),
}

PINS = [
    pins.test_worked_example_block_of_two,
    pins.test_worked_example_two_tiles_interview,
    lambda: pins.test_uniform_scores_give_mean_of_visible_values(True, 5, 9),
    lambda: pins.test_uniform_scores_give_mean_of_visible_values(True, 9, 5),
    lambda: pins.test_uniform_scores_give_mean_of_visible_values(2, 5, 9),
    lambda: pins.test_brute_force_tiny(2, 13, 4, 2),
    pins.test_rows_of_p_sum_to_one_and_are_nonnegative,
    lambda: pins.test_common_shift_cancels_and_guards_overflow(1e4),
    pins.test_special_cases,
    lambda: pins.test_brute_force_tiny(True, 3, 11, 8),
    lambda: pins.test_brute_force_tiny(False, 5, 5, 3),
    lambda: pins.test_torch_sdpa_float64(True),
    pins.test_bf16_inputs_are_widened_exactly,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
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


def test_unmutated_source_passes_every_pin():
    for pin in PINS:
        pin()
