"""Pins of the oracle's additive bias against facts that do not come from the oracle.

The bias is added to the scaled scores before the softmax ("Explain FlashAttention ...",
section "Keep only the state needed for the final weighted average"). Each test below
names what pins it: the pages' worked example rebuilt from a bias, a closed-form
equivalence with an extra coordinate, the causal mask as a -inf bias, shift invariance,
pure-Python brute force and the library routine. test_oracle_bias_mutants.py checks
that plausible slips in the bias code fail at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return {e["id"]: e for e in json.load(f)["examples"]}


def _num(x):
    return math.log(2.0) if x == "ln2" else float(x)


def _d1_bias(scores, values, scale, qk_part=None):
    """d=1 heads whose scaled score q*k_j*scale is qk_part[j] (0 if None) and whose bias
    fills the rest up to scores[j]."""
    n = len(scores)
    a = np.zeros(n) if qk_part is None else np.asarray(qk_part, np.float64)
    q = torch.ones((1, 1, 1, 1), dtype=torch.float64)
    k = torch.tensor(a / scale, dtype=torch.float64).view(1, 1, n, 1)
    v = torch.tensor(values, dtype=torch.float64).view(1, 1, n, 1)
    b = torch.tensor(np.asarray(scores, np.float64) - a, dtype=torch.float64).view(1, 1, 1, n)
    return q, k, v, b


@pytest.mark.parametrize("key", ["fa_optimization_worked_example", "fa_optimization_active_recall_1",
                                 "io_aware_interview_two_tiles"])
@pytest.mark.parametrize("split", [False, True])
def test_bias_rebuilds_the_worked_examples(key, split):
    """The worked examples of "Flash Attention Optimization" (section "Worked example:
    online softmax by hand", its "Active recall" question 1) and of the interview page
    (two tiles), with every score given as bias (split=False: q.k = 0) or half from the
    scaled q.k and half from the bias (split=True): the printed O must come out."""
    ex = _golden()[key]
    scale = 0.37
    s = [_num(x) for x in ex["scores"]]
    q, k, v, b = _d1_bias(s, [_num(x) for x in ex["values"]], scale, [x / 2 for x in s] if split else None)
    o, lse, p = oracle.attention(q, k, v, scale, bias=b, want_p=True)
    val, tol = ex["O_program_output"] if "O_program_output" in ex else ex["O"]
    assert abs(o[0, 0] - val) <= tol
    m = max(s)
    assert abs(lse[0] - (m + math.log(sum(math.exp(x - m) for x in s)))) <= 1e-12
    if "direct" in ex:
        w, tol = ex["direct"]["weights"]
        assert np.max(np.abs(p[0] - np.array(w))) <= tol


def _rand(shape, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * mult)


@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("Nq,Nk", [(5, 9), (9, 5), (7, 7)])
def test_rank_one_bias_equals_an_extra_coordinate(causal, Nq, Nk):
    """Closed form: a bias scale * a_i * c_j is the same as appending a_i to every query
    and c_j to every key (the scaled score gains exactly that product). a and c differ per
    (b, h), so a bias read with the wrong orientation, row or head does not match."""
    B, H, d, scale = 2, 3, 6, 0.41
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, H, Nk, d), 2), _rand((B, H, Nk, d), 3)
    a, c = _rand((B, H, Nq, 1), 4, 2.0), _rand((B, H, Nk, 1), 5, 2.0)
    bias = scale * a * c.transpose(2, 3)                       # [B, H, Nq, Nk]
    o1, l1 = oracle.attention(q, k, v, scale, causal, bias=bias)
    v0 = torch.cat([v, torch.zeros_like(c)], 3)                 # values gain a zero column
    o2, l2 = oracle.attention(torch.cat([q, a], 3), torch.cat([k, c], 3), v0, scale, causal)
    assert np.all(o2[:, d] == 0)
    o2 = o2[:, :d]
    fin = np.isfinite(l2)
    assert np.array_equal(fin, np.isfinite(l1))
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1[fin] - l2[fin])) <= 1e-13


@pytest.mark.parametrize("causal", [1, 2])
@pytest.mark.parametrize("Nq,Nk", [(6, 11), (11, 6), (8, 8)])
def test_neg_inf_bias_is_the_causal_mask(causal, Nq, Nk):
    """A bias of -inf on exactly the pairs the causal mask hides gives the causal result
    (the mask is one kind of additive bias); with Nq > Nk some rows see no key and must
    follow the empty-row policy (O = 0, LSE = -inf)."""
    B, H, d, scale = 1, 2, 5, 0.5
    q, k, v = _rand((B, H, Nq, d), 11), _rand((B, H, Nk, d), 12), _rand((B, H, Nk, d), 13)
    off = (Nk - Nq) if causal == 1 else 0
    i = torch.arange(Nq).view(-1, 1)
    j = torch.arange(Nk).view(1, -1)
    bias = torch.where(j <= i + off, 0.0, -math.inf).to(torch.float64)   # [Nq, Nk]
    o1, l1 = oracle.attention(q, k, v, scale, 0, bias=bias)
    o2, l2 = oracle.attention(q, k, v, scale, causal)
    assert np.array_equal(l1 == -np.inf, l2 == -np.inf)
    fin = np.isfinite(l2)
    assert np.max(np.abs(o1 - o2)) <= 1e-14
    assert np.max(np.abs(l1[fin] - l2[fin])) <= 1e-14
    if Nq > Nk and causal == 1:
        assert np.all(o1[:Nq - Nk] == 0) and np.all(l1[:Nq - Nk] == -np.inf)


def test_row_constant_bias_shifts_lse_only():
    """Softmax ignores a constant added to a whole row: O is unchanged and the log-sum-exp
    moves by that constant (bias of shape [B, H, Nq, 1], broadcast over the keys)."""
    B, H, Nq, Nk, d, scale = 2, 2, 7, 10, 4, 0.3
    q, k, v = _rand((B, H, Nq, d), 21), _rand((B, H, Nk, d), 22), _rand((B, H, Nk, d), 23)
    c = _rand((B, H, Nq, 1), 24, 50.0)
    o1, l1 = oracle.attention(q, k, v, scale, 1, bias=c)
    o2, l2 = oracle.attention(q, k, v, scale, 1)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - (l2 + c.reshape(-1).numpy()))) <= 1e-12


def _brute(q, k, v, scale, causal, bias):
    """Pure-Python attention with math.exp and math.fsum, no max subtraction (|s| small)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    off = (Nk - Nq) if causal == 1 else 0
    bb = bias.to(torch.float64).expand(B, H, Nq, Nk)
    O = np.zeros((B * H * Nq, d))
    L = np.full((B * H * Nq,), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                r = (b * H + h) * Nq + i
                w = []
                for j in range(Nk):
                    if causal and j > i + off:
                        w.append(0.0)
                        continue
                    s = scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d))
                    w.append(math.exp(s + float(bb[b, h, i, j])))
                tot = math.fsum(w)
                if tot == 0:
                    continue
                L[r] = math.log(tot)
                for t in range(d):
                    O[r, t] = math.fsum(w[j] * float(v[b, h, j, t]) for j in range(Nk)) / tot
    return O, L


@pytest.mark.parametrize("shape", [(1, 1, 5, 8), (5, 8), (3, 1, 8), (2, 1, 1, 8), (2, 3, 5, 8)])
@pytest.mark.parametrize("bdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [0, 1, 2])
def test_bias_brute_force_tiny(shape, bdtype, causal):
    """Independent pure-Python evaluation for every broadcast shape of the bias, float32
    and bfloat16 bias values, all three mask settings (Nq = 5, Nk = 8)."""
    B, H, Nq, Nk, d, scale = 2, 3, 5, 8, 3, 0.7
    q = _rand((B, H, Nq, d), 31).to(torch.float32)
    k = _rand((B, H, Nk, d), 32).to(torch.float32)
    v = _rand((B, H, Nk, d), 33).to(torch.float32)
    bias = _rand(shape, 34, 2.0).to(bdtype)
    o, l = oracle.attention(q, k, v, scale, causal, bias=bias)
    ob, lb = _brute(q, k, v, scale, causal, bias)
    assert np.array_equal(np.isfinite(l), np.isfinite(lb))
    assert np.max(np.abs(o - ob)) <= 1e-13
    fin = np.isfinite(lb)
    assert np.max(np.abs(l[fin] - lb[fin])) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_bias_matches_sdpa_float64(causal):
    """The library routine: torch's scaled_dot_product_attention in float64 on the CPU
    adds a float attn_mask to the scaled scores; with is_causal the mask is combined by
    hand (SDPA takes one or the other)."""
    B, H, N, d, scale = 2, 3, 13, 8, 0.35
    q, k, v = _rand((B, H, N, d), 41), _rand((B, H, N, d), 42), _rand((B, H, N, d), 43)
    bias = _rand((1, H, N, N), 44, 3.0)
    mask = bias
    if causal:
        mask = bias + torch.full((N, N), -math.inf, dtype=torch.float64).triu(1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    o, _ = oracle.attention(q, k, v, scale, causal, bias=bias)
    assert np.max(np.abs(o - ref.reshape(-1, d).numpy())) <= 1e-13


def test_broadcast_bias_equals_materialised_bias():
    """A bias broadcast with stride 0 reads the same values as the same bias written out
    in full."""
    B, H, Nq, Nk, d, scale = 3, 2, 6, 9, 4, 0.6
    q, k, v = _rand((B, H, Nq, d), 51), _rand((B, H, Nk, d), 52), _rand((B, H, Nk, d), 53)
    bias = _rand((1, H, 1, Nk), 54)
    o1, l1 = oracle.attention(q, k, v, scale, 1, bias=bias)
    o2, l2 = oracle.attention(q, k, v, scale, 1, bias=bias.expand(B, H, Nq, Nk).contiguous())
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_bias_rejects_bad_shapes():
    q = torch.zeros((1, 2, 3, 4))
    k = torch.zeros((1, 2, 5, 4))
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, k, 1.0, bias=torch.zeros((3, 3, 5)))   # H=3 against 2
    with pytest.raises(TypeError):
        oracle.attention(q, k, k, 1.0, bias=torch.zeros((3, 5), dtype=torch.int32))
