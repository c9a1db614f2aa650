"""Pins of the float64 backward oracle with an additive bias (CPU only).

The bias enters the scores as in the forward ("Explain FlashAttention ...", section "Keep
only the state needed for the final weighted average": scores are scaled, then the mask or
bias is added): S = scale * Q K^T + bias. Its gradients are those of that definition. They
are pinned here against things other than the oracle's formulas:
- central finite differences, in float64, of the forward oracle's loss sum(O * dO) with
  respect to q, k, v and bias entries;
- torch.autograd in float64 on CPU through an explicit softmax attention;
- closed forms: a zero bias gives the unbiased gradients exactly; a bias constant along
  each query row leaves dQ, dK and dV unchanged; -inf on the pairs the causal mask hides
  reproduces the causal gradients; every row of dBias sums to zero (the softmax Jacobian
  annihilates constants) and dBias is zero where a pair is hidden;
- a broadcast bias: finite differences of the shared parameter equal the full dBias summed
  over the broadcast dimensions.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _inputs(B, H, Nq, Nk, d, seed):
    return (_rand((B, H, Nq, d), seed), _rand((B, H, Nk, d), seed + 1),
            _rand((B, H, Nk, d), seed + 2), _rand((B, H, Nq, d), seed + 3))


def _loss(q, k, v, do, bias, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal, bias=bias)
    return float((o * do.reshape(-1, q.shape[-1]).numpy()).sum())


@pytest.mark.parametrize("causal,Nq,Nk", [(0, 5, 7), (1, 6, 6), (1, 4, 9), (2, 4, 9), (1, 9, 4)])
def test_finite_differences_with_bias(causal, Nq, Nk):
    B, H, d, scale = 1, 2, 4, 0.7
    q, k, v, do = _inputs(B, H, Nq, Nk, d, 21)
    bias = _rand((B, H, Nq, Nk), 25, 1.5)
    dq, dk, dv, db = oracle.attention_bwd(q, k, v, do, scale, causal, bias=bias, want_dbias=True)
    grads = {"q": dq, "k": dk, "v": dv, "bias": db}
    h = 1e-6
    rng = np.random.default_rng(9)
    for name, t in (("q", q), ("k", k), ("v", v), ("bias", bias)):
        flat = t.view(-1)
        for e in rng.choice(flat.numel(), size=12, replace=False):
            orig = float(flat[e])
            flat[e] = orig + h
            lp = _loss(q, k, v, do, bias, scale, causal)
            flat[e] = orig - h
            lm = _loss(q, k, v, do, bias, scale, causal)
            flat[e] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name].reshape(-1)[e]) <= 1e-7 * max(1.0, abs(fd)), (name, e)


def _torch_reference(q, k, v, do, bias, scale, causal):
    """dq, dk, dv, dbias by torch.autograd through an explicit softmax attention."""
    q, k, v, bias = (t.clone().requires_grad_(True) for t in (q, k, v, bias))
    s = scale * (q @ k.transpose(-1, -2)) + bias
    Nq, Nk = s.shape[-2:]
    if causal:
        off = Nk - Nq if causal == 1 else 0
        hide = torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None] + off
        s = s.masked_fill(hide, float("-inf"))
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)   # rows with no visible key: P = 0
    (p @ v * do).sum().backward()
    return q.grad, k.grad, v.grad, bias.grad


@pytest.mark.parametrize("causal,Nq,Nk,d", [(0, 17, 23, 16), (1, 33, 33, 8), (2, 20, 31, 8),
                                             (1, 30, 12, 8)])
def test_matches_torch_autograd_float64(causal, Nq, Nk, d):
    B, H, scale = 2, 3, 1 / math.sqrt(d)
    q, k, v, do = _inputs(B, H, Nq, Nk, d, 31)
    bias = _rand((B, H, Nq, Nk), 35, 2.0)
    got = oracle.attention_bwd(q, k, v, do, scale, causal, bias=bias, want_dbias=True)
    ref = _torch_reference(q, k, v, do, bias, scale, causal)
    for g, r in zip(got, ref):
        r = r.detach().numpy().reshape(g.shape)
        assert np.abs(g - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


def test_zero_bias_is_the_unbiased_backward_exactly():
    q, k, v, do = _inputs(2, 2, 40, 50, 8, 41)
    for causal in (0, 1, 2):
        a = oracle.attention_bwd(q, k, v, do, 0.3, causal)
        b = oracle.attention_bwd(q, k, v, do, 0.3, causal, bias=torch.zeros(40, 50, dtype=torch.float64))
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_row_constant_bias_leaves_qkv_gradients():
    q, k, v, do = _inputs(1, 2, 30, 30, 8, 51)
    rowc = _rand((1, 2, 30, 1), 55, 3.0)
    a = oracle.attention_bwd(q, k, v, do, 0.4, 1)
    b = oracle.attention_bwd(q, k, v, do, 0.4, 1, bias=rowc, want_dbias=True)
    for x, y in zip(a, b[:3]):
        assert np.abs(x - y).max() <= 1e-12 * np.abs(x).max()


def test_dbias_rows_sum_to_zero_and_vanish_where_hidden():
    Nq, Nk = 25, 30
    q, k, v, do = _inputs(2, 2, Nq, Nk, 8, 61)
    bias = _rand((2, 2, Nq, Nk), 65, 2.0)
    bias[0, 1, 3, :] = -math.inf           # a row whose keys are all hidden
    bias[1, 0, :, 7] = -math.inf           # a key hidden from every row
    for causal in (0, 1, 2):
        *_, db = oracle.attention_bwd(q, k, v, do, 0.5, causal, bias=bias, want_dbias=True)
        db = db.reshape(2, 2, Nq, Nk)
        assert np.abs(db.sum(-1)).max() <= 1e-12 * max(1.0, np.abs(db).max())
        assert np.all(db[0, 1, 3, :] == 0.0) and np.all(db[1, 0, :, 7] == 0.0)
        if causal:
            off = Nk - Nq if causal == 1 else 0
            hide = np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off
            assert np.all(db[:, :, hide] == 0.0)


def test_minus_inf_bias_on_hidden_pairs_equals_causal():
    Nq, Nk = 20, 28
    q, k, v, do = _inputs(1, 2, Nq, Nk, 8, 71)
    hide = torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None] + (Nk - Nq)
    mask_bias = torch.zeros(Nq, Nk, dtype=torch.float64).masked_fill(hide, -math.inf)
    a = oracle.attention_bwd(q, k, v, do, 0.6, 1)
    b = oracle.attention_bwd(q, k, v, do, 0.6, 0, bias=mask_bias)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12 * np.abs(x).max()


@pytest.mark.parametrize("shape", [(1, 1, 9, 11), (2, 1, 1, 11), (1, 2, 9, 11)])
def test_broadcast_bias_gradient_is_the_sum(shape):
    """A bias shared along some dimensions: its gradient is the full dBias summed over them
    (finite differences of the shared parameter)."""
    B, H, Nq, Nk, d, scale = 2, 2, 9, 11, 4, 0.8
    q, k, v, do = _inputs(B, H, Nq, Nk, d, 81)
    bias = _rand(shape, 85, 1.0)
    *_, db = oracle.attention_bwd(q, k, v, do, scale, 1, bias=bias, want_dbias=True)
    db = db.reshape(B, H, Nq, Nk)
    dims = tuple(i for i in range(4) if shape[i] == 1 and (B, H, Nq, Nk)[i] > 1)
    want = db.sum(axis=dims, keepdims=True)
    h = 1e-6
    flat = bias.view(-1)
    for e in range(0, flat.numel(), max(1, flat.numel() // 10)):
        orig = float(flat[e])
        flat[e] = orig + h
        lp = _loss(q, k, v, do, bias, scale, 1)
        flat[e] = orig - h
        lm = _loss(q, k, v, do, bias, scale, 1)
        flat[e] = orig
        fd = (lp - lm) / (2 * h)
        assert abs(fd - want.reshape(-1)[e]) <= 1e-7 * max(1.0, abs(fd)), e


def test_dbias_needs_every_row():
    q, k, v, do = _inputs(1, 1, 5, 5, 4, 91)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, v, do, 0.5, 0, qrows=[0, 1], bias=torch.zeros(5, 5),
                             want_dbias=True)
