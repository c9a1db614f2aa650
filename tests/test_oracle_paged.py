"""Pins of the paged-cache oracle (CPU only).

oracle.paged_attention gathers each sequence's logical key/value rows through its block
table and applies the attention definition. It is pinned against things other than its
own gather:
- a cache built here, by explicit loops, from contiguous [B, H, N, d] tensors with an
  identity table, and then with the pages shuffled in the pool, must reproduce
  oracle.attention on the contiguous tensors;
- a sequence length below the table's capacity equals attention over that prefix;
- the worked example of "Flash Attention Optimization" (scores 1, 3, 2, 5 over values
  10, 20, 30, 40 give 36.880565891447), laid out over two pages in reverse order;
- a sequence with no key gives O = 0 and LSE = -inf; a page id outside the pool holds no
  keys (those positions are left out).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _build_cache(k, page_size, order):
    """k [B, H, N, d] -> (cache [B*P, ps, H, d], table [B, P]) with page (b, p) stored at
    pool slot order[b*P + p]; written with plain loops, not with the oracle's gather."""
    B, H, N, d = k.shape
    P = math.ceil(N / page_size)
    cache = torch.zeros((B * P, page_size, H, d), dtype=k.dtype)
    table = torch.zeros((B, P), dtype=torch.int32)
    for b in range(B):
        for p in range(P):
            slot = int(order[b * P + p])
            table[b, p] = slot
            for t in range(page_size):
                n = p * page_size + t
                if n < N:
                    for h in range(H):
                        cache[slot, t, h] = k[b, h, n]
    return cache, table


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_paged_matches_contiguous(dtype, page_size):
    g = torch.Generator().manual_seed(3)
    B, H, N, d = 3, 2, 37, 8
    q = (torch.randn((B, H, 1, d), generator=g) * 2).to(dtype)
    k = (torch.randn((B, H, N, d), generator=g) * 2).to(dtype)
    v = torch.randn((B, H, N, d), generator=g).to(dtype)
    P = math.ceil(N / page_size)
    want_o, want_l = oracle.attention(q, k, v, 0.3, False)
    for order in (np.arange(B * P), np.random.default_rng(1).permutation(B * P)):
        kc, table = _build_cache(k, page_size, order)
        vc, _ = _build_cache(v, page_size, order)
        o, l = oracle.paged_attention(q, kc, vc, table, [N] * B, page_size, 0.3)
        assert np.max(np.abs(o - want_o)) <= 1e-14 and np.max(np.abs(l - want_l)) <= 1e-14


def test_paged_prefix_lengths_and_empty_sequence():
    g = torch.Generator().manual_seed(4)
    B, H, N, d, ps = 4, 3, 40, 5, 8
    q = torch.randn((B, H, 1, d), generator=g)
    k = torch.randn((B, H, N, d), generator=g)
    v = torch.randn((B, H, N, d), generator=g)
    order = np.random.default_rng(2).permutation(B * 5)
    kc, table = _build_cache(k, ps, order)
    vc, _ = _build_cache(v, ps, order)
    lens = [0, 1, 17, 40]
    o, l = oracle.paged_attention(q, kc, vc, table, lens, ps, 0.5)
    for b, n in enumerate(lens):
        rows = slice(b * H, (b + 1) * H)
        if n == 0:
            assert np.all(o[rows] == 0) and np.all(np.isneginf(l[rows]))
            continue
        wo, wl = oracle.attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.5, False)
        assert np.max(np.abs(o[rows] - wo)) <= 1e-14 and np.max(np.abs(l[rows] - wl)) <= 1e-14


def test_paged_worked_example_two_pages_reversed():
    """d = 1: q = [1], k_j = [s_j], scale 1; keys 0-1 sit in pool page 1, keys 2-3 in page 0."""
    ex = json.load(open(GOLDEN))
    case = next(c for c in ex["examples"] if c["id"] == "fa_optimization_worked_example")
    s, vals = case["scores"], case["values"]
    want, tol = case["O_program_output"]
    kc = torch.tensor([[[[s[2]]], [[s[3]]]], [[[s[0]]], [[s[1]]]]], dtype=torch.float64).float()
    vc = torch.tensor([[[[vals[2]]], [[vals[3]]]], [[[vals[0]]], [[vals[1]]]]], dtype=torch.float64).float()
    q = torch.ones((1, 1, 1, 1))
    o, l = oracle.paged_attention(q, kc, vc, torch.tensor([[1, 0]]), [4], 2, 1.0)
    assert abs(o[0, 0] - want) <= tol


def test_page_outside_pool_holds_no_keys():
    g = torch.Generator().manual_seed(5)
    H, d, ps = 2, 4, 4
    kc = torch.randn((3, ps, H, d), generator=g)
    vc = torch.randn((3, ps, H, d), generator=g)
    q = torch.randn((1, H, 1, d), generator=g)
    o, l = oracle.paged_attention(q, kc, vc, torch.tensor([[2, 7, -1, 0]]), [14], ps, 0.4)
    # positions 0-3 come from page 2, 4-11 from invalid pages (left out), 12-13 from page 0
    k_log = torch.cat([kc[2], kc[0, :2]], 0).permute(1, 0, 2)[None]
    v_log = torch.cat([vc[2], vc[0, :2]], 0).permute(1, 0, 2)[None]
    wo, wl = oracle.attention(q, k_log.contiguous(), v_log.contiguous(), 0.4, False)
    assert np.max(np.abs(o - wo)) <= 1e-14 and np.max(np.abs(l - wl)) <= 1e-14
