"""GPU parity of the float32 backward pass (fa_bwd with FA_F32) against the float64 oracle.

O and LSE come from the float32 forward, as in training. Tolerance, derived from the
arithmetic: nothing is rounded below float32, so the error is float32 rounding in the
score, probability and gradient contractions plus that of the forward's O and LSE. A float32
evaluation of the same formulas (tests/tolerance_model.py, checked by
tests/test_tolerance_model.py: P recomputed from the float32 LSE of a float32 online-softmax
forward) stays within 6.0e-6 * max|g*| (max error) and 3.2e-6 * mean|g*| (mean error)
against the oracle on shapes from 128 to 2048 rows, d = 64 and 128, with and without the
causal mask and with Q, K scaled up to x3. The bounds are about three times that, for each
of dQ, dK, dV:
    max|g - g*| <= 2e-5 * max|g*|        mean|g - g*| <= 1e-5 * mean|g*|
A gradient that is zero in exact arithmetic (dQ and dK when no query row sees more than one
key) is pure float32 rounding residue, of the size of a few ulps of the case's other
gradients; only for such a gradient are max|g*| and mean|g*| replaced by 0.1 times the
case's largest gradient (a residue of up to 2e-6 of it, ~30 float32 ulps, is accepted).
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import workloads as W
from parity_util import BWD_F32_MAX_REL, BWD_F32_MEAN_REL, finite_scale, say, seeded
from test_bwd_parity import _all_rows

pytestmark = pytest.mark.gpu

F32_BOUNDS = dict(max_rel=BWD_F32_MAX_REL, mean_rel=BWD_F32_MEAN_REL, floor_frac=0.1)
PAIRS = [(1, 1), (17, 17), (31, 33), (64, 64), (65, 65), (127, 129), (129, 127), (1, 300),
         (300, 1), (17, 200), (200, 17), (64, 300), (300, 64), (257, 255)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _run(q, k, v, do, scale, causal):
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["full", "bottom_right", "top_left"])
def test_bwd_f32_edge_grid(d, causal):
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(PAIRS):
        what = f"f32 backward d={d} causal={causal} Nq={nq} Nk={nk}"
        say(what)
        q = seeded((2, 2, nq, d), 3100 + idx, torch.float32, mult=2.0)
        k = seeded((2, 2, nk, d), 3200 + idx, torch.float32, mult=2.0)
        v = seeded((2, 2, nk, d), 3300 + idx, torch.float32)
        do = seeded((2, 2, nq, d), 3400 + idx, torch.float32)
        dq, dk, dv = _run(q, k, v, do, scale, causal)
        _all_rows(q, k, v, do, scale, causal, dq, dk, dv, what, **F32_BOUNDS)


def test_bwd_f32_workload1_shape():
    """The float32 workload's shape (B=1, H=1, N=256, d=64, not causal) with its inputs and a
    seeded dO, all rows."""
    w = W.WORKLOADS[1]
    say("f32 backward on the float32 workload's shape")
    q, k, v = W.make_inputs(w, "cuda")
    do = W.make_grad(w, "cuda")
    dq, dk, dv = _run(q, k, v, do, w.scale, w.causal)
    st = _all_rows(q, k, v, do, w.scale, w.causal, dq, dk, dv, "workload 1 backward", **F32_BOUNDS)
    say(f"  {st}")


def test_bwd_f32_larger_causal():
    """Many tiles per workgroup and a sharp softmax: B=1, H=3, N=1000, d=128, Q and K x3."""
    q = seeded((1, 3, 1000, 128), 3501, torch.float32, mult=3.0)
    k = seeded((1, 3, 1000, 128), 3502, torch.float32, mult=3.0)
    v = seeded((1, 3, 1000, 128), 3503, torch.float32)
    do = seeded((1, 3, 1000, 128), 3504, torch.float32)
    say("f32 backward N=1000 causal")
    dq, dk, dv = _run(q, k, v, do, finite_scale(128), True)
    st = _all_rows(q, k, v, do, finite_scale(128), True, dq, dk, dv, "f32 N=1000", **F32_BOUNDS)
    say(f"  {st}")


def test_bwd_f32_overwrites_outputs_and_is_deterministic():
    q = seeded((2, 3, 150, 64), 3601, torch.float32)
    k = seeded((2, 3, 130, 64), 3602, torch.float32)
    v = seeded((2, 3, 130, 64), 3603, torch.float32)
    do = seeded((2, 3, 150, 64), 3604, torch.float32)
    o, lse = fa.fwd(q, k, v, causal=True)
    outs = []
    for _ in range(2):
        dq = torch.full((2, 3, 150, 64), float("nan"), device="cuda")
        dk = torch.full((2, 3, 130, 64), float("nan"), device="cuda")
        dv = torch.full((2, 3, 130, 64), float("nan"), device="cuda")
        ws = torch.full((fa.bwd_workspace_bytes(2, 3, 150),), 255, dtype=torch.uint8, device="cuda")
        say("f32 backward NaN-prefilled outputs")
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert torch.isfinite(t).all()
        outs.append((dq, dk, dv))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_bwd_f32_rows_that_see_no_key_get_zero_gradient():
    """Causal with Nq > Nk: the first Nq - Nk query rows see no key (LSE = -inf)."""
    q = seeded((1, 2, 90, 64), 3701, torch.float32)
    k = seeded((1, 2, 40, 64), 3702, torch.float32)
    v = seeded((1, 2, 40, 64), 3703, torch.float32)
    do = seeded((1, 2, 90, 64), 3704, torch.float32)
    say("f32 backward empty rows")
    dq, dk, dv = _run(q, k, v, do, 0.125, 1)
    assert torch.all(dq[:, :, :50] == 0)
    _all_rows(q, k, v, do, 0.125, 1, dq, dk, dv, "f32 empty rows", **F32_BOUNDS)
