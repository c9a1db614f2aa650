"""The derived tolerances of the GPU parity tests, reproduced on the CPU.

For gradients and for 8-bit inputs no bound is stated, so the parity tests derive theirs
from the kernels' arithmetic: tests/tolerance_model.py performs the kernels' roundings in
float32 and is compared here with the float64 oracle. Each test checks the model's worst
error over its cases against the figure the parity test's docstring quotes, and that the
parity test's bound leaves the stated margin above it. For the bfloat16 forward, whose
bounds are stated, the model shows they hold with margin, and that O rounded to bfloat16
on output would not hold them (the reason O is float32).
"""
import pytest
import torch

import tolerance_model as M
from parity_util import (BF16_LSE_MAX, BF16_O_MAX, BF16_O_MEAN, BWD_BF16_MAX_REL,
                         BWD_BF16_MEAN_REL, BWD_F32_MAX_REL, BWD_F32_MEAN_REL, FP8_O_MAX,
                         FP8_O_MEAN)

# (B, H, Nq, Nk, d, causal, Q/K factor, seed): every mask setting, Nq != Nk both ways, rows
# that see no key (Nq > Nk, bottom-right), the sharp x3 inputs of the N = 8192 workload
BWD_CASES = [(1, 2, 256, 256, 64, 0, 1.0, 1), (1, 2, 256, 256, 128, 1, 3.0, 2),
             (1, 2, 1000, 1000, 128, 1, 1.0, 3), (1, 1, 2048, 2048, 64, 0, 1.0, 4),
             (1, 1, 2048, 2048, 128, 1, 3.0, 5), (1, 2, 300, 128, 64, 1, 2.0, 6),
             (1, 2, 128, 300, 128, 1, 2.0, 7), (1, 2, 500, 500, 128, 2, 2.0, 8)]


def _worst(cases, **kw):
    wmax = wmean = 0.0
    for c in cases:
        for emax, emean in M.bwd_case(*c, **kw).values():
            wmax, wmean = max(wmax, emax), max(wmean, emean)
    return wmax, wmean


def test_bwd_bf16_model_and_bounds():
    wmax, wmean = _worst(BWD_CASES)
    # the figures quoted in test_bwd_parity.py
    assert wmax <= 3.0e-3 and wmean <= 1.8e-3, (wmax, wmean)
    # and the model is not trivially exact: bfloat16 operands leave ~2^-9 relative error
    assert wmean >= 5e-4
    assert BWD_BF16_MAX_REL >= 3.0 * wmax and BWD_BF16_MEAN_REL >= 2.5 * wmean


def test_bwd_f32_model_and_bounds():
    wmax, wmean = _worst(BWD_CASES[:6], dtype=torch.float32)
    assert wmax <= 6.0e-6 and wmean <= 3.2e-6, (wmax, wmean)
    assert BWD_F32_MAX_REL >= 3.0 * wmax and BWD_F32_MEAN_REL >= 3.0 * wmean


E4M3_CASES = [(1, 4, 512, 128, 0, 1.0, 1), (1, 4, 2048, 128, 1, 3.0, 2),
              (1, 2, 2048, 128, 1, 1.0, 3), (1, 2, 4096, 128, 1, 3.0, 5),
              (2, 2, 300, 128, 1, 2.0, 6), (2, 3, 1000, 128, 0, 2.0, 7)]


def test_e4m3_model_and_bounds():
    wmax = wmean = 0.0
    for c in E4M3_CASES:
        emax, emean = M.e4m3_case(*c)
        wmax, wmean = max(wmax, emax), max(wmean, emean)
    assert wmax <= 0.070 and wmean <= 0.0039, (wmax, wmean)
    assert FP8_O_MAX >= 1.7 * wmax and FP8_O_MEAN >= 1.5 * wmean
    # the worst case 2^-4 * max|V| (~0.3 for N(0,1) values) is far looser than the bound
    assert FP8_O_MAX <= 0.5 * 2.0 ** -4 * 4.0


@pytest.mark.parametrize("case", [(1, 2, 2048, 128, 1, 3.0, 11), (1, 2, 4096, 128, 1, 3.0, 12),
                                  (1, 4, 2048, 64, 0, 1.0, 13)])
def test_fwd_bf16_model_within_stated_bounds(case):
    omax, omean, lmax, omax_bf16_out = M.fwd_case(*case)
    assert omax <= 0.5 * BF16_O_MAX and omean <= 0.1 * BF16_O_MEAN and lmax <= 0.1 * BF16_LSE_MAX
    if case[5] == 3.0:
        # sharp softmax: O close to one V row of size up to ~5, where a bfloat16 output's
        # half-ulp (2^-8 of the value) alone exceeds the 1e-2 bound
        assert omax_bf16_out > BF16_O_MAX


def test_model_exact_when_nothing_is_rounded():
    """Guard on the models themselves: without the bfloat16 roundings the float32 model of
    the forward agrees with the oracle to float32 rounding, so what the bounds above measure
    is the roundings and not a flaw of the model."""
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn((1, 2, 300, 64), generator=g) for _ in range(3))
    o, lse = M.fwd_bf16(q, k, v, 0.125, 1, round_p=False)
    import oracle
    o_ref, l_ref = oracle.attention(q, k, v, 0.125, 1)
    assert float((o.double().reshape(o_ref.shape) - torch.from_numpy(o_ref)).abs().max()) <= 2e-6
    assert float((lse.double().reshape(-1) - torch.from_numpy(l_ref)).abs().max()) <= 2e-6
