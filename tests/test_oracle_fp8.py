"""Pins of the oracle path for 8-bit inputs (CPU only).

E4M3 inputs reach the oracle as float64 tensors holding value * descale exactly (a 4-bit
significand times a float32 factor fits in a double). Pinned here:
- the float64 input path is the float32 path: identical results on the same values;
- the decode of E4M3 bytes (torch.float8_e4m3fn) against values fixed by the format's
  definition (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0,
  the all-ones pattern NaN, no infinities);
- the worked example of "Flash Attention Optimization" (scores 1, 3, 2, 5 over values
  10, 20, 30, 40: O = 36.880565891447), all of whose numbers are exact in E4M3, through the
  8-bit encode / decode;
- descale factors enter linearly: q and k scaled by a and 1/a (both powers of two) change
  nothing.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")

# (byte, value) from the E4M3 definition: value = (-1)^s * 2^(e-7) * (1 + m/8), e > 0;
# (-1)^s * 2^-6 * (m/8) for e = 0; 0x7f / 0xff are NaN.
E4M3 = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5),
        (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x44, 3.0), (0x4A, 5.0),
        (0x52, 10.0), (0x5A, 20.0), (0x5F, 30.0), (0x62, 40.0), (0x77, 240.0), (0x78, 256.0),
        (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)]


def test_e4m3_decode_matches_the_format_definition():
    b = torch.tensor([x for x, _ in E4M3], dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = b.to(torch.float64).tolist()
    assert got == [v for _, v in E4M3]
    nan = torch.tensor([0x7F, 0xFF], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    assert torch.isnan(nan).all()
    # and the encode of those values returns the same bytes
    enc = torch.tensor([v for _, v in E4M3], dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8)
    assert enc.tolist() == [x for x, _ in E4M3]


@pytest.mark.parametrize("causal", [False, True])
def test_float64_path_equals_float32_path(causal):
    g = torch.Generator().manual_seed(9)
    q, k, v = (torch.randn((2, 3, 17, 8), generator=g) for _ in range(3))
    a = oracle.attention(q, k, v, 0.4, causal)
    b = oracle.attention(q.double(), k.double(), v.double(), 0.4, causal)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_worked_example_through_e4m3():
    ex = json.load(open(GOLDEN))
    case = next(c for c in ex["examples"] if c["id"] == "fa_optimization_worked_example")
    want, tol = case["O_program_output"]
    enc = lambda x: torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn)
    q8 = enc([[[[1.0]]]])
    k8 = enc([[[[s] for s in case["scores"]]]])
    v8 = enc([[[[x] for x in case["values"]]]])
    dec = lambda t: t.to(torch.float64)
    o, _ = oracle.attention(dec(q8), dec(k8), dec(v8), 1.0, False)
    assert abs(o[0, 0] - want) <= tol


def test_descales_enter_linearly():
    g = torch.Generator().manual_seed(10)
    x = [torch.randn((1, 2, 40, 16), generator=g).to(torch.float8_e4m3fn) for _ in range(3)]
    q, k, v = (t.to(torch.float64) for t in x)
    a = oracle.attention(q * 4.0, k * 0.25, v, 0.3, True)
    b = oracle.attention(q, k, v, 0.3, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
