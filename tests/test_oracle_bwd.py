"""Pins of the float64 backward oracle (CPU only).

The pages describe the backward pass only as recomputing the probability tiles
from the saved row statistics ("Flash Attention Optimization", section "Sizing
a tile, and why the backward pass recomputes instead of storing"); the
gradients are those of the forward definition. They are pinned here against
things other than the oracle's own formulas:
- central finite differences of the forward oracle's loss sum(O * dO);
- torch.autograd in float64 on CPU (a library routine);
- invariants that hold for any input: sum_j dK_j = 0 (every softmax row's
  Jacobian annihilates constants), sum_j dV_j = sum_i dO_i over rows that see a
  key (rows of P sum to 1);
- closed forms: equal value rows give dQ = dK = 0; one key gives dQ = dK = 0 and
  dV_0 = sum_i dO_i; dO = 0 gives zero gradients; a row with no visible key
  contributes nothing.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).float()


def _inputs(B, H, Nq, Nk, d, seed=0, qk=1.0):
    return (_rand((B, H, Nq, d), seed, qk), _rand((B, H, Nk, d), seed + 1, qk),
            _rand((B, H, Nk, d), seed + 2), _rand((B, H, Nq, d), seed + 3))


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float((o * do.double().reshape(-1, q.shape[-1]).numpy()).sum())


@pytest.mark.parametrize("causal,Nq,Nk", [(False, 5, 7), (True, 6, 6), (True, 4, 9), (2, 4, 9), (2, 9, 4)])
def test_finite_differences(causal, Nq, Nk):
    B, H, d, scale = 1, 2, 4, 0.7
    q, k, v, do = _inputs(B, H, Nq, Nk, d, seed=11)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    grads = {"q": dq, "k": dk, "v": dv}
    h = 2.0 ** -12  # exact in float32 for these magnitudes; truncation error O(h^2)
    rng = np.random.default_rng(5)
    for name, t in (("q", q), ("k", k), ("v", v)):
        flat = t.view(-1)
        for e in rng.choice(flat.numel(), size=12, replace=False):
            orig = float(flat[e])
            flat[e] = orig + h
            lp = _loss(q, k, v, do, scale, causal)
            flat[e] = orig - h
            lm = _loss(q, k, v, do, scale, causal)
            flat[e] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name].reshape(-1)[e]) <= 1e-6 * max(1.0, abs(fd)), (name, e)


def _autograd(q, k, v, do, scale, causal):
    qq, kk, vv = [x.double().clone().requires_grad_() for x in (q, k, v)]
    s = qq @ kk.transpose(-1, -2) * scale
    Nq, Nk = q.shape[2], k.shape[2]
    if causal:
        mask = torch.arange(Nk)[None, :] > (torch.arange(Nq)[:, None] + (Nk - Nq))
        s = s.masked_fill(mask, float("-inf"))
    o = torch.softmax(s, -1) @ vv
    (o * do.double()).sum().backward()
    d = q.shape[-1]
    return [x.grad.reshape(-1, d).numpy() for x in (qq, kk, vv)]


@pytest.mark.parametrize("causal,Nq,Nk,d", [(False, 33, 47, 16), (True, 40, 40, 8),
                                            (True, 17, 50, 32), (False, 1, 64, 64)])
def test_matches_torch_autograd_float64(causal, Nq, Nk, d):
    q, k, v, do = _inputs(2, 3, Nq, Nk, d, seed=21, qk=1.5)
    scale = 1 / math.sqrt(d)
    got = oracle.attention_bwd(q, k, v, do, scale, causal)
    ref = _autograd(q, k, v, do, scale, causal)
    for g, r in zip(got, ref):
        assert np.abs(g - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, N, d = 2, 2, 24, 8
    q, k, v, do = _inputs(B, H, N, N, d, seed=31, qk=2.0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, causal)
    dk = dk.reshape(B * H, N, d)
    dv = dv.reshape(B * H, N, d)
    dof = do.double().reshape(B * H, N, d).numpy()
    assert np.abs(dk.sum(axis=1)).max() <= 1e-12
    assert np.abs(dv.sum(axis=1) - dof.sum(axis=1)).max() <= 1e-12


def test_equal_value_rows_give_no_score_gradient():
    q, k, _, do = _inputs(1, 2, 9, 13, 8, seed=41)
    v = _rand((1, 2, 1, 8), 99).expand(1, 2, 13, 8).contiguous()
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.3, False)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    # O = v_0 for every row, so dV_j = sum_i P_ij dO_i still needs P: check its total
    assert np.allclose(dv.reshape(2, 13, 8).sum(1), do.double().sum(2).reshape(2, 8).numpy(),
                       atol=1e-12)


def test_single_key_and_zero_upstream():
    q, k, v, do = _inputs(1, 1, 6, 1, 4, seed=51)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() <= 1e-15
    assert np.allclose(dv[0], do.double()[0, 0].sum(0).numpy(), atol=1e-14)
    z = torch.zeros_like(do)
    dq, dk, dv = oracle.attention_bwd(q, k, v, z, 0.5, False)
    assert not np.any(dq) and not np.any(dk) and not np.any(dv)


def test_empty_rows_contribute_nothing():
    # causal with Nq > Nk: query rows 0 .. Nq-Nk-1 see no key
    B, H, Nq, Nk, d = 1, 1, 10, 4, 8
    q, k, v, do = _inputs(B, H, Nq, Nk, d, seed=61)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True)
    empty = Nq - Nk
    assert not np.any(dq[:empty])
    do2 = do.clone()
    do2[:, :, :empty] = 0
    q2 = q.clone()
    q2[:, :, :empty] = 7.0  # whatever an empty row holds does not matter
    _, dk2, dv2 = oracle.attention_bwd(q2, k, v, do2, 0.5, True)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_sampled_rows_equal_full_result():
    q, k, v, do = _inputs(2, 2, 20, 30, 8, seed=71)
    full = oracle.attention_bwd(q, k, v, do, 0.5, True)
    qrows = [0, 7, 19, 20, 39, 75]
    krows = [0, 29, 30, 44, 119]
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True, qrows=qrows, krows=krows)
    assert np.array_equal(dq, full[0][qrows])
    assert np.array_equal(dk, full[1][krows]) and np.array_equal(dv, full[2][krows])
