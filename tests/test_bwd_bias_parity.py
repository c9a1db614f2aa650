"""GPU parity of the biased backward pass (fa_bwd_bias) against the float64 oracle
(oracle.attention_bwd with the same bias).

O and LSE come from fa_fwd_bias, as in training. dQ, dK and dV are judged with the bounds
of the unbiased bfloat16 backward (test_bwd_parity.py: P and dS are bfloat16 MFMA operands,
everything else float32; the bias only adds one float32 fma per score):
    max|g - g*| <= 1e-2 * max|g*|        mean|g - g*| <= 5e-3 * mean|g*|
dBias is dS in float32, written before any rounding to bfloat16; its error comes from O
(through rowsum(dO * O), whose bfloat16-P rounding the forward leaves) and is of the same
relative size, so it is judged with the same bounds.
"""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
import workloads as W
from parity_util import finite_scale, rows_of, say, seeded
from test_bwd_parity import compare_grads, exact_zero_grads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _run(q, k, v, bias, do, scale, causal, want_dbias=True):
    o, lse = fa.fwd_bias(q, k, v, bias, scale=scale, causal=causal)
    out = fa.bwd_bias(q, k, v, bias, o, lse, do, scale=scale, causal=causal, want_dbias=want_dbias)
    torch.cuda.synchronize()
    return out


def _check_all(q, k, v, bias, do, scale, causal, got, what):
    d = q.shape[-1]
    ref = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), scale, causal, bias=bias.cpu(),
                               want_dbias=True)
    names = ("dq", "dk", "dv", "dbias")
    g = {n: t.cpu().numpy().reshape(-1, d if n != "dbias" else k.shape[2]) for n, t in zip(names, got)}
    r = dict(zip(names, ref))
    zero = exact_zero_grads(q.shape[2], k.shape[2], causal)
    st = compare_grads({n: g[n] for n in names[:3]}, {n: r[n] for n in names[:3]}, what, zero=zero)
    if zero:
        # every row sees at most one key: dS is zero in exact arithmetic and the kernels'
        # float32 residue is judged against 1e-2 of the case's largest gradient
        floor = 1e-2 * max(float(np.abs(r[n]).max()) for n in names[:3])
        assert np.abs(r["dbias"]).max() == 0.0
        assert float(np.abs(g["dbias"]).max()) <= 1e-2 * floor, f"{what}: dbias residue"
    else:
        st.update({("dbias" if n == "dv" else n): x for n, x in
                   compare_grads({"dv": g["dbias"]}, {"dv": r["dbias"]}, what + " dbias").items()})
    return st


PAIRS = [(1, 1), (17, 17), (31, 33), (63, 64), (65, 65), (127, 129), (129, 127), (200, 200),
         (1, 300), (300, 1), (64, 300), (300, 64), (257, 255)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["full", "bottom_right", "top_left"])
def test_bwd_bias_edge_grid(d, causal):
    """A full bias (N(0,1) x 2, some keys and one row hidden by -inf) at ragged sizes around
    every tile edge, Nq != Nk both ways; dQ, dK, dV and dBias against the oracle."""
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(PAIRS):
        say(f"bwd bias d={d} causal={causal} Nq={nq} Nk={nk}")
        B, H = 2, 2
        q = seeded((B, H, nq, d), 5000 + idx, torch.bfloat16, mult=2.0)
        k = seeded((B, H, nk, d), 5100 + idx, torch.bfloat16, mult=2.0)
        v = seeded((B, H, nk, d), 5200 + idx, torch.bfloat16)
        do = seeded((B, H, nq, d), 5300 + idx, torch.bfloat16)
        bias = seeded((B, H, nq, nk), 5400 + idx, torch.bfloat16, mult=2.0)
        if nk > 3:
            bias[0, 1, :, nk // 3] = -math.inf
        if nq > 3 and nk > 1:
            bias[1, 0, nq // 2, :] = -math.inf
        bias = fa.pad_bias(bias)
        got = _run(q, k, v, bias, do, scale, causal)
        st = _check_all(q, k, v, bias, do, scale, causal, got, f"Nq={nq} Nk={nk}")
        say(f"  {st}")


@pytest.mark.parametrize("shape", [(2, 1, 1, 333), (1, 1, 250, 333), (1, 3, 250, 333)],
                         ids=["key_padding", "shared", "per_head"])
def test_bwd_bias_broadcast(shape):
    """Biases shared along some dimensions (stride 0): dQ, dK, dV against the oracle with the
    same broadcast bias; dBias is the full-layout dS, which the oracle returns too."""
    B, H, nq, nk, d = 2, 3, 250, 333, 128
    q = seeded((B, H, nq, d), 5501, torch.bfloat16, mult=2.0)
    k = seeded((B, H, nk, d), 5502, torch.bfloat16, mult=2.0)
    v = seeded((B, H, nk, d), 5503, torch.bfloat16)
    do = seeded((B, H, nq, d), 5504, torch.bfloat16)
    bias = fa.pad_bias(seeded(shape, 5505, torch.bfloat16, mult=2.0))
    for causal in (0, 1):
        say(f"bwd bias broadcast {shape} causal={causal}")
        got = _run(q, k, v, bias, do, finite_scale(d), causal)
        st = _check_all(q, k, v, bias, do, finite_scale(d), causal, got, f"{shape} causal={causal}")
        say(f"  {st}")


def test_bwd_bias_zero_matches_unbiased_and_deterministic():
    """A zero bias gives the unbiased backward's gradients up to rounding order; two calls
    agree bit for bit and overwrite NaN-filled outputs everywhere (dBias included, also the
    pairs the causal mask skips)."""
    B, H, nq, nk, d = 2, 2, 300, 517, 128
    q = seeded((B, H, nq, d), 5601, torch.bfloat16, mult=2.0)
    k = seeded((B, H, nk, d), 5602, torch.bfloat16, mult=2.0)
    v = seeded((B, H, nk, d), 5603, torch.bfloat16)
    do = seeded((B, H, nq, d), 5604, torch.bfloat16)
    zero = fa.pad_bias(torch.zeros((nq, nk), dtype=torch.bfloat16, device=DEV))
    for causal in (0, 1, 2):
        say(f"bwd bias zero causal={causal}")
        o, lse = fa.fwd(q, k, v, causal=causal)
        ref = fa.bwd(q, k, v, o, lse, do, causal=causal)
        runs = []
        for _ in range(2):
            outs = [torch.full(s, float("nan"), device=DEV) for s in
                    ((B, H, nq, d), (B, H, nk, d), (B, H, nk, d), (B, H, nq, nk))]
            fa.bwd_bias(q, k, v, zero, o, lse, do, causal=causal, dq=outs[0], dk=outs[1], dv=outs[2],
                        dbias=outs[3])
            torch.cuda.synchronize()
            assert not any(torch.isnan(t).any() for t in outs)
            runs.append(outs)
        assert all(torch.equal(a, b) for a, b in zip(*runs))
        for a, b in zip(runs[0][:3], ref):
            assert float((a - b).abs().max()) <= 2e-3 * float(b.abs().max())
        if causal:
            off = nk - nq if causal == 1 else 0
            hide = torch.arange(nk, device=DEV)[None, :] > torch.arange(nq, device=DEV)[:, None] + off
            assert not runs[0][3][:, :, hide].any()


def test_bwd_bias_workload3_sampled():
    """The causal N = 8192 workload with its full [B, H, N, N] bias, in the launch
    configuration the benchmark times: dQ on sampled rows, dK and dV on sampled rows of two
    heads (dBias not requested)."""
    w = W.WORKLOADS[3]
    say(f"bwd bias workload: {w.name} with a full bias")
    q, k, v = W.make_inputs(w, DEV)
    do = W.make_grad(w, DEV)
    bias = W.make_bias(w, DEV)
    dq, dk, dv = _run(q, k, v, bias, do, w.scale, True, want_dbias=False)
    BH = w.B * w.H
    qrows = W.sample_rows(w, 32)
    kw = W.Workload(w.number, w.name, w.B, w.H, w.Nk, w.Nk, w.d, w.dtype, w.causal)
    krows = [int(r) for r in W.sample_rows(kw, 48) if r // w.Nk in (0, BH - 1)]
    say(f"  oracle: {len(qrows)} dQ rows, {len(krows)} dK/dV rows")
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), w.scale, True,
                                      qrows=qrows, krows=krows, bias=bias.cpu())
    got = {"dq": rows_of(dq, qrows, w.d), "dk": rows_of(dk, krows, w.d), "dv": rows_of(dv, krows, w.d)}
    st = compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, "bias workload")
    say(f"  {st}")


def test_bwd_bias_rejects():
    q = seeded((1, 1, 8, 64), 5701, torch.bfloat16)
    o = torch.zeros((1, 1, 8, 64), device=DEV)
    lse = torch.zeros((1, 1, 8), device=DEV)
    bias = fa.pad_bias(torch.zeros((8, 8), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(NotImplementedError):       # float32 inputs are not offered here
        fa.bwd_bias(q.float(), q.float(), q.float(), bias.float(), o, lse, q.float())
    with pytest.raises(ValueError):                # a mis-sized dbias
        fa.bwd_bias(q, q, q, bias, o, lse, q, dbias=torch.zeros((1, 1, 8, 9), device=DEV))
