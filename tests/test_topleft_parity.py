"""GPU parity of the top-left causal alignment (causal = 2: query i sees key j iff j <= i)
against the float64 oracle, for the prefill (bfloat16 and float32), the packed
variable-length prefill and the backward pass, at the bounds of each path's own tests."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from parity_util import compare, finite_scale, oracle_rows, say, seeded
from test_bwd_parity import _all_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [(1, 300), (17, 1000), (64, 65), (65, 64), (128, 300), (300, 128), (257, 129),
         (1000, 17), (48, 1000), (255, 256), (16, 15), (200, 200)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_topleft_prefill(dtype, d):
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(PAIRS):
        say(f"top-left {dtype} d={d} Nq={nq} Nk={nk}")
        q = seeded((2, 3, nq, d), 1100 + idx, dtype, mult=2.0)
        k = seeded((2, 3, nk, d), 1200 + idx, dtype, mult=2.0)
        v = seeded((2, 3, nk, d), 1300 + idx, dtype)
        o, lse = fa.fwd(q, k, v, scale=scale, causal=2)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_rows(q, k, v, scale, 2)
        compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref, dtype,
                f"top-left Nq={nq} Nk={nk}")


def test_topleft_equals_bottom_right_when_square():
    q = seeded((2, 4, 500, 128), 1401, torch.bfloat16, mult=2.0)
    k = seeded((2, 4, 500, 128), 1402, torch.bfloat16, mult=2.0)
    v = seeded((2, 4, 500, 128), 1403, torch.bfloat16)
    say("top-left vs bottom-right, Nq = Nk")
    a = fa.fwd(q, k, v, causal=1)
    b = fa.fwd(q, k, v, causal=2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
def test_topleft_backward(d):
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate([(64, 300), (300, 64), (17, 1000), (1000, 17), (257, 129)]):
        say(f"top-left backward d={d} Nq={nq} Nk={nk}")
        q = seeded((1, 2, nq, d), 1500 + idx, torch.bfloat16, mult=2.0)
        k = seeded((1, 2, nk, d), 1510 + idx, torch.bfloat16, mult=2.0)
        v = seeded((1, 2, nk, d), 1520 + idx, torch.bfloat16)
        do = seeded((1, 2, nq, d), 1530 + idx, torch.bfloat16)
        o, lse = fa.fwd(q, k, v, scale=scale, causal=2)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=scale, causal=2)
        torch.cuda.synchronize()
        _all_rows(q, k, v, do, scale, 2, dq, dk, dv, f"top-left Nq={nq} Nk={nk}")


def test_topleft_varlen():
    H, d = 3, 128
    nqs, nks = [300, 17, 512, 1], [200, 400, 700, 5]
    cq = torch.tensor([0] + list(np.cumsum(nqs)), dtype=torch.int32)
    ck = torch.tensor([0] + list(np.cumsum(nks)), dtype=torch.int32)
    q = seeded((int(cq[-1]), H, d), 1601, torch.bfloat16, mult=2.0)
    k = seeded((int(ck[-1]), H, d), 1602, torch.bfloat16, mult=2.0)
    v = seeded((int(ck[-1]), H, d), 1603, torch.bfloat16)
    say("top-left varlen")
    o, lse = fa.fwd_varlen(q, k, v, cq.to(DEV), ck.to(DEV), max(nqs), scale=0.1, causal=2)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q.cpu(), k.cpu(), v.cpu(), cq.tolist(), ck.tolist(), 0.1, 2)
    compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().T.reshape(-1), o_ref.reshape(-1, d),
            l_ref.T.reshape(-1), torch.bfloat16, "top-left varlen")
