"""The bias pins must catch plausible slips in the oracle's bias code: each mutant is a
copy of the oracle source with one planted mistake, compiled on the CPU, and at least one
pin of test_oracle_bias.py has to fail against it. Every mutant keeps all memory accesses
in bounds.
"""
import os
import subprocess

import pytest
import torch

import oracle
import test_oracle_bias as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
ADD = "if (bias && bias->p) s[j] += widen(bias->p, bias->dtype, brow + (size_t)j);"

MUTANTS = {
    "bias subtracted": (ADD, ADD.replace("s[j] +=", "s[j] -=")),
    "bias multiplied by the scale": (ADD, ADD.replace("s[j] += widen", "s[j] += scale * widen")),
    "bias dropped": (ADD, ADD.replace("if (bias && bias->p)", "if (0)")),
    "bias row of query 0 for every query": ("(long long)i * bias->sq);", "0LL * bias->sq);"),
    "bias ignores the batch index": ("brow = (size_t)((bh / H) * bias->sb", "brow = (size_t)(0 * bias->sb"),
    "bias ignores the head index": ("(bh / H) * bias->sb + (bh % H) * bias->sh + (long long)i * bias->sq);",
                                    "(bh / H) * bias->sb + 0 * bias->sh + (long long)i * bias->sq);"),
    "bias also un-hides masked keys": (
        "if ((long long)j > last_visible) { s[j] = -INFINITY; continue; }",
        "if ((long long)j > last_visible && !(bias && bias->p)) { s[j] = -INFINITY; continue; }"),
}

PINS = [
    lambda: pins.test_bias_rebuilds_the_worked_examples("fa_optimization_worked_example", False),
    lambda: pins.test_bias_rebuilds_the_worked_examples("fa_optimization_worked_example", True),
    lambda: pins.test_rank_one_bias_equals_an_extra_coordinate(1, 5, 9),
    lambda: pins.test_rank_one_bias_equals_an_extra_coordinate(0, 9, 5),
    lambda: pins.test_neg_inf_bias_is_the_causal_mask(1, 11, 6),
    pins.test_row_constant_bias_shifts_lse_only,
    lambda: pins.test_bias_brute_force_tiny((2, 3, 5, 8), torch.float32, 1),
    lambda: pins.test_bias_matches_sdpa_float64(True),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bias_pins_catch_mutant(name, tmp_path, monkeypatch):
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


def test_unmutated_source_passes_every_bias_pin():
    for pin in PINS:
        pin()
