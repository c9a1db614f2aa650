"""The bias-backward pins must catch plausible slips: each mutant is a copy of the oracle
source with one planted mistake in the bias path of the gradient code, compiled on the CPU,
and at least one pin in test_oracle_bwd_bias.py has to fail against it. Every mutant keeps
all memory accesses in bounds.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_bwd_bias as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
BIAS_ADD = ("    sc += widen(bias->p, bias->dtype,\n"
            "                (size_t)((bh / H) * bias->sb + (bh % H) * bias->sh + (long long)i * bias->sq + j));")

MUTANTS = {
    "bias left out of the recomputed scores": (BIAS_ADD, "    (void)H;"),
    "bias multiplied by the scale": (
        BIAS_ADD,
        BIAS_ADD.replace("sc += widen(", "sc += scale * widen(")),
    "bias subtracted": (BIAS_ADD, BIAS_ADD.replace("sc += widen(", "sc -= widen(")),
    "bias of the key's row instead of the query's": (
        BIAS_ADD, BIAS_ADD.replace("(long long)i * bias->sq + j", "(long long)j * bias->sq + i")),
    "row statistics without the bias": (
        "  one_row(q, k, v, dtype, H, Nq, Nk, d, scale, causal, bias, r, s, o, lse, NULL);",
        "  one_row(q, k, v, dtype, H, Nq, Nk, d, scale, causal, NULL, r, s, o, lse, NULL);"),
    "dBias = P instead of dS": ("        if (grow) grow[j] = ds;", "        if (grow) grow[j] = p;"),
    "dBias scaled like dQ": ("        if (grow) grow[j] = ds;", "        if (grow) grow[j] = scale * ds;"),
}

PINS = [
    lambda: pins.test_finite_differences_with_bias(1, 4, 9),
    lambda: pins.test_finite_differences_with_bias(0, 5, 7),
    lambda: pins.test_matches_torch_autograd_float64(2, 20, 31, 8),
    pins.test_zero_bias_is_the_unbiased_backward_exactly,
    pins.test_row_constant_bias_leaves_qkv_gradients,
    pins.test_dbias_rows_sum_to_zero_and_vanish_where_hidden,
    pins.test_minus_inf_bias_on_hidden_pairs_equals_causal,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bias_bwd_pins_catch_mutant(name, tmp_path, monkeypatch):
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


def test_unmutated_source_passes_every_bias_bwd_pin():
    for pin in PINS:
        pin()
