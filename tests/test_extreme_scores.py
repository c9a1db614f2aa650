"""GPU parity at the degenerate ends of the softmax: scores of magnitude ~500 (a large scale:
every row is dominated by a few keys, and exp(s) of the raw scores would overflow float32
many times over; larger scores would leave float32 score rounding of ~1e-3 in the LSE, the
size of its bound, in any float32 implementation), scores of magnitude ~1e-5 (a tiny scale: the weights are uniform to float32
precision, O is the mean of the visible values and LSE = ln(count)), and rows whose scores
all tie. Prefill in both dtypes and both mask settings, the split-KV decode and the backward
pass, each against the float64 oracle at the bounds of the other parity tests.
"""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from parity_util import compare, say, seeded
from test_bwd_parity import compare_grads, exact_zero_grads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _f32(x):
    return float(torch.tensor(x, dtype=torch.float32).item())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("scale", [20.0, 1e-6], ids=["sharp", "flat"])
def test_prefill_extreme_scale(dtype, d, causal, scale):
    """At the sharp end the float32 path is held to the absolute bounds of the bfloat16
    path, not to 1e-5 of max|O*|: float32 scores of magnitude ~1e3 carry rounding of ~1e-4,
    which moves the weights of near-tied keys by that relative amount in any float32
    implementation (measured: ~1e-4 on O)."""
    B, H, nq, nk = 1, 2, 200, 333
    sc = _f32(scale)
    say(f"extreme prefill {dtype} d={d} causal={causal} scale={sc}")
    q = seeded((B, H, nq, d), 9101, dtype)
    k = seeded((B, H, nk, d), 9102, dtype)
    v = seeded((B, H, nk, d), 9103, dtype)
    o, lse = fa.fwd(q, k, v, scale=sc, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), sc, causal)
    bounds = torch.bfloat16 if scale > 1 else dtype
    st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), ro, rl, bounds,
                 f"scale {sc}")
    say(f"  {st}")
    if scale < 1e-3:
        # uniform weights: LSE = ln(visible keys) up to the tiny scores
        counts = np.array([min(nk, i + nk - nq + 1) if causal else nk for i in range(nq)] * (B * H))
        assert np.abs(lse.cpu().numpy().reshape(-1) - np.log(counts)).max() <= 1e-3


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_all_scores_tie(dtype):
    """q = k = the same row for every position: every visible score is equal, so O is the
    mean of the visible values whatever the scale (here 3: scores ~380)."""
    B, H, nq, nk, d = 1, 1, 150, 260, 128
    row = seeded((1, 1, 1, d), 9111, dtype)
    q = row.expand(B, H, nq, d).contiguous()
    k = row.expand(B, H, nk, d).contiguous()
    v = seeded((B, H, nk, d), 9112, dtype)
    for causal in (0, 1):
        say(f"tied scores {dtype} causal={causal}")
        o, lse = fa.fwd(q, k, v, scale=3.0, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), 3.0, causal)
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), ro, rl, dtype,
                     "ties")
        vf = v.double().cpu().numpy().reshape(nk, d)
        for i in (0, nq // 2, nq - 1):
            n = min(nk, i + nk - nq + 1) if causal else nk
            assert np.abs(ro[i] - vf[:n].mean(0)).max() <= 1e-12
        say(f"  {st}")


@pytest.mark.parametrize("scale", [20.0, 1e-6], ids=["sharp", "flat"])
def test_decode_extreme_scale(scale):
    B, H, nk, d = 2, 3, 5000, 128
    sc = _f32(scale)
    say(f"extreme decode scale={sc}")
    q = seeded((B, H, 1, d), 9121, torch.bfloat16)
    k = seeded((B, H, nk, d), 9122, torch.bfloat16)
    v = seeded((B, H, nk, d), 9123, torch.bfloat16)
    o, lse = fa.decode(q, k, v, num_splits=16, scale=sc)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), sc, 0)
    st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), ro, rl,
                 torch.bfloat16, f"decode scale {sc}")
    say(f"  {st}")


@pytest.mark.parametrize("scale", [0.5, 1e-6], ids=["sharp", "flat"])
@pytest.mark.parametrize("causal", [0, 1])
def test_backward_extreme_scale(scale, causal):
    """Gradients at a sharp softmax (scores ~6 apart: most of each row's weight on a few
    keys) and a flat one (uniform to float32 precision); bounds of the bfloat16 backward
    relative to each gradient's own size (at the flat end dQ and dK are ~scale times dV).
    The saturated end is left out: there dQ and dK vanish in exact arithmetic while dP - D
    keeps float32 rounding of dP's size, so no bound relative to their own size can hold."""
    B, H, nq, nk, d = 1, 2, 190, 260, 128
    sc = _f32(scale)
    say(f"extreme backward scale={sc} causal={causal}")
    q = seeded((B, H, nq, d), 9131, torch.bfloat16)
    k = seeded((B, H, nk, d), 9132, torch.bfloat16)
    v = seeded((B, H, nk, d), 9133, torch.bfloat16)
    do = seeded((B, H, nq, d), 9134, torch.bfloat16)
    o, lse = fa.fwd(q, k, v, scale=sc, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=sc, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), sc, causal)
    got = {n: t.cpu().numpy().reshape(-1, d) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    st = compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, f"scale {sc}",
                       zero=exact_zero_grads(nq, nk, causal))
    say(f"  {st}")
    assert math.isfinite(float(dq.abs().max())) and math.isfinite(float(dk.abs().max()))
