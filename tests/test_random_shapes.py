"""Seeded random shapes through every entry point, each compared on all rows with the float64
oracle at the bounds of the dedicated parity tests. The shapes, scales, value spreads and
mask modes are drawn from fixed seeds, so a failure names a case that reruns identically."""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from parity_util import compare, say, seeded
from test_bwd_parity import _all_rows
from test_bwd_f32_parity import F32_BOUNDS

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _f32(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).item())


def _len(rng, lo, hi):
    """Log-uniform integer in [lo, hi]: short and long sizes equally often."""
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def _case(rng, max_pairs):
    d = int(rng.choice([64, 128]))
    while True:
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        nq, nk = _len(rng, 1, 700), _len(rng, 1, 700)
        if B * H * nq * nk <= max_pairs:
            break
    causal = int(rng.integers(0, 3))
    scale = _f32(rng.uniform(0.3, 1.5) / math.sqrt(d))
    mult = float(rng.uniform(0.5, 3.0))
    return B, H, nq, nk, d, causal, scale, mult


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_random_forward(dtype):
    rng = np.random.default_rng(7001 if dtype == torch.bfloat16 else 7002)
    for c in range(16):
        B, H, nq, nk, d, causal, scale, mult = _case(rng, 1_500_000)
        what = f"fwd {dtype} case {c}: B={B} H={H} Nq={nq} Nk={nk} d={d} causal={causal} scale={scale:.4f}"
        say(what)
        q = seeded((B, H, nq, d), 9000 + 3 * c, dtype, mult=mult)
        k = seeded((B, H, nk, d), 9001 + 3 * c, dtype, mult=mult)
        v = seeded((B, H, nk, d), 9002 + 3 * c, dtype)
        o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, causal)
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref,
                     l_ref, dtype, what)
        say(f"  {st}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_random_bias(dtype):
    """Bias shapes drawn among full, per-head, shared and key-padding broadcasts, with -inf
    entries hiding random keys."""
    rng = np.random.default_rng(7011 if dtype == torch.bfloat16 else 7012)
    for c in range(10):
        B, H, nq, nk, d, causal, scale, mult = _case(rng, 1_000_000)
        causal = min(causal, 1)
        form = ["full", "per_head", "shared", "key_padding"][int(rng.integers(0, 4))]
        shape = {"full": (B, H, nq, nk), "per_head": (1, H, nq, nk), "shared": (1, 1, nq, nk),
                 "key_padding": (B, 1, 1, nk)}[form]
        what = (f"bias {dtype} case {c}: B={B} H={H} Nq={nq} Nk={nk} d={d} causal={causal} "
                f"bias={form}")
        say(what)
        q = seeded((B, H, nq, d), 9100 + 4 * c, dtype, mult=mult)
        k = seeded((B, H, nk, d), 9101 + 4 * c, dtype, mult=mult)
        v = seeded((B, H, nk, d), 9102 + 4 * c, dtype)
        bias = seeded(shape, 9103 + 4 * c, torch.float32, mult=2.0)
        hide = torch.from_numpy(rng.random(shape) < 0.1).to(DEV)
        bias = bias.masked_fill(hide, float("-inf")).to(dtype)
        full = bias.expand(B, H, nq, nk)
        arg = fa.pad_bias(bias) if dtype == torch.bfloat16 else bias  # broadcast by strides
        o, lse = fa.fwd_bias(q, k, v, arg, scale=scale, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, causal,
                                        bias=full.contiguous().cpu())
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref,
                     l_ref, dtype, what)
        say(f"  {st}")


def test_random_varlen():
    rng = np.random.default_rng(7021)
    for c in range(8):
        d = int(rng.choice([64, 128]))
        H = int(rng.integers(1, 5))
        nb = int(rng.integers(1, 7))
        lq = [_len(rng, 1, 600) for _ in range(nb)]
        lk = [_len(rng, 1, 600) if rng.random() < 0.5 else n for n in lq]
        causal = int(rng.integers(0, 3))
        scale = _f32(rng.uniform(0.3, 1.5) / math.sqrt(d))
        what = f"varlen case {c}: H={H} d={d} causal={causal} lq={lq} lk={lk}"
        say(what)
        cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
        ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
        q = seeded((int(cq[-1]), H, d), 9200 + 3 * c, torch.bfloat16, mult=2.0)
        k = seeded((int(ck[-1]), H, d), 9201 + 3 * c, torch.bfloat16, mult=2.0)
        v = seeded((int(ck[-1]), H, d), 9202 + 3 * c, torch.bfloat16)
        o, lse = fa.fwd_varlen(q, k, v, cq.to(DEV), ck.to(DEV), max(lq), scale=scale,
                               causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_varlen(q.cpu(), k.cpu(), v.cpu(), cq.tolist(),
                                               ck.tolist(), scale, causal)
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().T.reshape(-1),
                     o_ref.reshape(-1, d), l_ref.T.reshape(-1), torch.bfloat16, what)
        say(f"  {st}")


def test_random_decode():
    rng = np.random.default_rng(7031)
    for c in range(8):
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        nk = _len(rng, 1, 20000)
        splits = int(rng.integers(1, 130))
        scale = _f32(rng.uniform(0.3, 1.5) / math.sqrt(d))
        what = f"decode case {c}: B={B} H={H} Nk={nk} d={d} splits={splits}"
        say(what)
        q = seeded((B, H, 1, d), 9300 + 3 * c, torch.bfloat16, mult=2.0)
        k = seeded((B, H, nk, d), 9301 + 3 * c, torch.bfloat16, mult=2.0)
        v = seeded((B, H, nk, d), 9302 + 3 * c, torch.bfloat16)
        o, lse = fa.decode(q, k, v, num_splits=splits, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, False)
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref,
                     l_ref, torch.bfloat16, what)
        say(f"  {st}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_random_backward(dtype):
    rng = np.random.default_rng(7041 if dtype == torch.bfloat16 else 7042)
    bounds = {} if dtype == torch.bfloat16 else F32_BOUNDS
    for c in range(8):
        B, H, nq, nk, d, causal, scale, mult = _case(rng, 600_000)
        what = f"bwd {dtype} case {c}: B={B} H={H} Nq={nq} Nk={nk} d={d} causal={causal}"
        say(what)
        q = seeded((B, H, nq, d), 9400 + 4 * c, dtype, mult=mult)
        k = seeded((B, H, nk, d), 9401 + 4 * c, dtype, mult=mult)
        v = seeded((B, H, nk, d), 9402 + 4 * c, dtype)
        do = seeded((B, H, nq, d), 9403 + 4 * c, dtype)
        o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
        torch.cuda.synchronize()
        st = _all_rows(q, k, v, do, scale, causal, dq, dk, dv, what, **bounds)
        say(f"  {st}")


def test_random_fp8():
    """E4M3 inputs with per-tensor descales, at the FP8 bounds of the FP8 parity tests."""
    from test_fp8_parity import _case as fp8_case
    rng = np.random.default_rng(7051)
    for c in range(8):
        B, H, nq, nk, _, causal, _, mult = _case(rng, 1_000_000)
        say(f"fp8 case {c}: B={B} H={H} Nq={nq} Nk={nk} causal={causal} mult={mult:.2f}")
        st = fp8_case(B, H, nq, nk, causal, 9500 + c, mult=mult)
        say(f"  {st}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_random_paged(dtype):
    """Random page sizes, per-sequence lengths (zero included) and chunk counts over a pool
    with pages in random order."""
    from test_paged_parity import _case as paged_case
    rng = np.random.default_rng(7061 if dtype == torch.bfloat16 else 7062)
    for c in range(8):
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 6)), int(rng.integers(1, 5))
        ps = int(rng.choice([1, 4, 16, 64, 128, 256]))
        lens = [0 if rng.random() < 0.1 else _len(rng, 1, 6000 if ps > 1 else 300)
                for _ in range(B)]
        S = int(rng.integers(1, 100))
        st = paged_case(B, H, d, ps, lens, S, dtype, 9600 + 10 * c)
        say(f"  {st}")
