"""GPU parity of the prefill with an additive bias (fa_fwd_bias) against the float64
oracle: every broadcast form of the bias, ragged sizes that cross tile edges, all three mask
settings, -inf biases that hide keys and whole rows, large-magnitude biases, and the
causal B=2 H=16 N=8192 d=128 workload with a full per-(b, h) bias on sampled rows."""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
import workloads as W
from parity_util import compare, finite_scale, rows_of, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [(1, 300), (17, 1000), (64, 65), (257, 129), (300, 333), (1000, 17), (200, 200)]
# bias shapes broadcast to [B, H, Nq, Nk] (B = 2, H = 3)
FORMS = ["full", "per_head", "shared", "key_padding"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _bias(form, B, H, nq, nk, seed, dtype):
    shape = {"full": (B, H, nq, nk), "per_head": (1, H, nq, nk), "shared": (nq, nk),
             "key_padding": (B, 1, 1, nk)}[form]
    b = seeded(shape, seed, dtype, mult=3.0)
    if form == "key_padding":  # batch 0 hides its last third of keys, batch 1 its first key
        b[0, ..., nk - nk // 3:] = -math.inf
        b[1, ..., :1] = -math.inf
    return b


def _check(q, k, v, bias, scale, causal, what):
    d = q.shape[-1]
    o, lse = fa.fwd_bias(q, k, v, fa.pad_bias(bias), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, causal, bias=bias.cpu())
    return compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                   q.dtype, what)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2])
def test_bias_prefill(dtype, d, causal):
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(PAIRS):
        form = FORMS[idx % len(FORMS)]
        what = f"bias {form} {dtype} d={d} causal={causal} Nq={nq} Nk={nk}"
        say(what)
        q = seeded((2, 3, nq, d), 2100 + idx, dtype, mult=2.0)
        k = seeded((2, 3, nk, d), 2200 + idx, dtype, mult=2.0)
        v = seeded((2, 3, nk, d), 2300 + idx, dtype)
        _check(q, k, v, _bias(form, 2, 3, nq, nk, 2400 + idx, dtype), scale, causal, what)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_bias_every_form_one_shape(dtype):
    d, nq, nk = 128, 333, 517
    for idx, form in enumerate(FORMS):
        what = f"bias form {form} {dtype}"
        say(what)
        q = seeded((2, 3, nq, d), 2500 + idx, dtype, mult=2.0)
        k = seeded((2, 3, nk, d), 2510 + idx, dtype, mult=2.0)
        v = seeded((2, 3, nk, d), 2520 + idx, dtype)
        _check(q, k, v, _bias(form, 2, 3, nq, nk, 2530 + idx, dtype), 0.09, 1, what)


def test_bias_alibi_and_row_shift():
    """Large-magnitude biases: a linear distance penalty -slope_h * |i - j| (slopes
    2^(-8(h+1)/H), values down to about -500) plus a per-row constant of +-1e3, which the
    softmax must cancel exactly (only the LSE moves; exp(1e3) overflows without the max
    subtraction). The constant stays near 1e3 because the LSE is a float32 output: at
    |LSE| ~ 1e4 one float32 ulp is already 1e-3, the LSE bound itself."""
    B, H, N, d = 1, 4, 1000, 128
    q = seeded((B, H, N, d), 2601, torch.bfloat16, mult=2.0)
    k = seeded((B, H, N, d), 2602, torch.bfloat16, mult=2.0)
    v = seeded((B, H, N, d), 2603, torch.bfloat16)
    i = torch.arange(N, device=DEV).view(-1, 1)
    j = torch.arange(N, device=DEV).view(1, -1)
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], device=DEV)
    shift = torch.where(i % 2 == 0, 1e3, -1e3).float()
    bias = (-(slopes.view(H, 1, 1) * (i - j).abs().float()) + shift).to(torch.bfloat16)[None]
    for causal in (0, 1):
        say(f"bias alibi causal={causal}")
        _check(q, k, v, bias, 1.0 / math.sqrt(d), causal, f"alibi causal={causal}")


def test_bias_hiding_whole_rows_gives_empty_rows():
    """A -inf bias on every key of some rows: those rows follow the empty-row policy
    (O = 0, LSE = -inf); with causal = 1 and Nq > Nk the mask empties more rows."""
    B, H, nq, nk, d = 1, 2, 300, 200, 64
    q = seeded((B, H, nq, d), 2701, torch.bfloat16)
    k = seeded((B, H, nk, d), 2702, torch.bfloat16)
    v = seeded((B, H, nk, d), 2703, torch.bfloat16)
    bias = seeded((B, H, nq, nk), 2704, torch.bfloat16)
    bias[:, :, 150:170] = -math.inf
    for causal in (0, 1):
        say(f"bias empty rows causal={causal}")
        st = _check(q, k, v, bias, 0.125, causal, f"empty rows causal={causal}")
        say(f"  {st}")


def test_bias_zero_matches_plain_prefill():
    """A zero bias gives the plain prefill's result up to rounding order (the biased kernel
    uses 64-key tiles)."""
    q = seeded((2, 4, 700, 128), 2801, torch.bfloat16, mult=2.0)
    k = seeded((2, 4, 700, 128), 2802, torch.bfloat16, mult=2.0)
    v = seeded((2, 4, 700, 128), 2803, torch.bfloat16)
    say("bias zero vs plain")
    a = fa.fwd(q, k, v, causal=1)
    b = fa.fwd_bias(q, k, v, torch.zeros((700, 704), dtype=torch.bfloat16, device=DEV)[:, :700],
                    causal=1)
    torch.cuda.synchronize()
    assert float((a[0] - b[0]).abs().max()) <= 4e-3
    assert float((a[1] - b[1]).abs().max()) <= 1e-4


def test_bias_rejects_unpadded_bf16_rows():
    """A bfloat16 bias whose 13-key rows are not padded to 16 elements is refused by the
    binding (the kernel reads rows in 16-byte pieces); pad_bias makes it acceptable."""
    q = seeded((1, 1, 16, 64), 2901, torch.bfloat16)
    k = seeded((1, 1, 13, 64), 2902, torch.bfloat16)
    v = seeded((1, 1, 13, 64), 2903, torch.bfloat16)
    bias = seeded((16, 13), 2904, torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd_bias(q, k, v, bias)
    say("bias padded 13-key rows")
    _check(q, k, v, bias, 0.125, 0, "padded 13-key rows")


def test_bias_workload_sampled():
    """Causal B=2 H=16 N=8192 d=128 (Q, K x3) with a full [B, H, N, N] bfloat16 bias
    (N(0,1) x 2), in the launch configuration the benchmark times; 64 sampled rows per head."""
    w = W.WORKLOADS[3]
    say("bias workload: causal B=2 H=16 N=8192 d=128 with a full bias (sampled rows)")
    q, k, v = W.make_inputs(w, DEV)
    bias = W.make_bias(w, DEV)
    o, lse = fa.fwd_bias(q, k, v, bias, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rows = W.sample_rows(w, 64)
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), w.scale, True, rows=rows,
                                    bias=bias.cpu())
    st = compare(rows_of(o, rows, w.d), rows_of(lse, rows), o_ref, l_ref, w.dtype, "bias workload")
    say(f"  {st}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_bias_overwrites_outputs_and_is_deterministic(dtype):
    """NaN-prefilled O and LSE are fully overwritten, and two calls agree bit for bit."""
    q = seeded((2, 3, 300, 128), 2951, dtype, mult=2.0)
    k = seeded((2, 3, 333, 128), 2952, dtype, mult=2.0)
    v = seeded((2, 3, 333, 128), 2953, dtype)
    bias = fa.pad_bias(_bias("full", 2, 3, 300, 333, 2954, dtype))
    outs = []
    for _ in range(2):
        o = torch.full((2, 3, 300, 128), float("nan"), device=DEV)
        lse = torch.full((2, 3, 300), float("nan"), device=DEV)
        say(f"bias NaN-prefilled outputs {dtype}")
        fa.fwd_bias(q, k, v, bias, causal=1, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and not torch.isnan(lse).any()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
